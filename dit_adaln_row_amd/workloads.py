"""The synthetic workloads the kernels are measured and checked on.

Each workload mirrors an activation shape the pages measure on (FLUX.1,
ERNIE-Image, GLM-Image, Wan 2.1 VAE) with seeded synthetic values of a stated
distribution; no model weights or datasets are involved.  This module holds
shapes, distributions and the algorithmic-byte model only -- none of the
method's arithmetic.

Algorithmic bytes of one launch = every input element read once + every
output element written once (bf16 = 2 B, fp32 = 4 B), modulation / weight /
bias rows counted once per launch, debug outputs off.  This is the byte model
under which the Wan page's "1.5 TB/s", "4.1 TB/s", "0.63 TB/s" and "~3 TB/s"
figures are reproduced from its millisecond timings ("Fuse the Wan VAE conv
bias epilogue and tile the RMSNorm+SiLU kernel", Motivation and "Speed Tests
and Profiling").
"""
from __future__ import annotations

from dataclasses import dataclass, field

BF16 = 2
F32 = 4


@dataclass(frozen=True)
class Tensor:
    """A generated tensor: shape, distribution N(mu, sigma), storage kind."""
    name: str
    shape: tuple
    mu: float
    sigma: float
    kind: str = "bf16"   # "bf16" | "f16" | "f32" | "f32_bf16vals" (fp32 holding bf16 values)


@dataclass(frozen=True)
class Launch:
    """One library call of a workload."""
    name: str            # workload-unique launch name
    entry: str           # library entry point
    rows: int
    cols: int
    inputs: tuple        # tensor names read
    eps: float
    n_mod_rows: int = 1  # modulation rows (B) for the batched sites
    extra: dict = field(default_factory=dict)

    def algorithmic_bytes(self) -> int:
        r, c = self.rows, self.cols
        if self.entry in ("ln_modulate", "ln_modulate_folded"):
            return 2 * r * c * BF16 + 2 * self.n_mod_rows * c * BF16
        if self.entry == "gated_ln_modulate":
            return 4 * r * c * BF16 + 3 * self.n_mod_rows * c * BF16
        if self.entry == "rms_modulate":
            gated = self.extra.get("gated", False)
            act = (4 if gated else 2) * r * c * BF16
            vec = c * BF16 + (3 if gated else 2) * self.n_mod_rows * c * BF16
            return act + vec
        if self.entry == "qk_layernorm":
            return 2 * r * c * BF16  # r counts q rows + k rows
        if self.entry == "rmsnorm_silu_bias":
            vec = (2 if self.extra.get("bias", True) else 1) * c * F32
            return 2 * r * c * BF16 + vec
        if self.entry == "conv_bias_epilogue":
            es = F32 if self.extra.get("dtype") == "f32" else BF16  # bf16 and fp16: 2 bytes
            bs = BF16 if self.extra.get("bias_dtype", "f32") != "f32" else F32
            act = (3 if self.extra.get("residual", False) else 2) * r * c * es
            return act + c * bs
        # standalone elementwise stages: bf16 and fp16 are both 2-byte types
        if self.entry == "modulate_scale_shift":
            return 2 * r * c * BF16 + 2 * self.n_mod_rows * c * BF16
        if self.entry == "residual_gate_add":
            return 3 * r * c * BF16 + self.n_mod_rows * c * BF16
        if self.entry == "ln_modulate_backward":
            # x and d_out read, d_x written, scale read, d_scale and d_shift written
            es = F32 if self.extra.get("dtype") == "f32" else BF16
            return 3 * r * c * es + self.n_mod_rows * c * (es + 2 * F32)
        raise KeyError(self.entry)

    def label(self) -> str:
        """The kernel kind a profiler trace attributes this launch to."""
        if self.entry == "rms_modulate" and self.extra.get("gated"):
            return "gated_rms_modulate"
        if self.entry in ("modulate_scale_shift", "residual_gate_add"):
            return f"{self.entry}_{self.extra.get('dtype', 'bf16')}"
        if self.entry == "conv_bias_epilogue" and self.extra.get("dtype", "bf16") != "bf16":
            return f"{self.entry}_{self.extra['dtype']}"
        return self.entry


def _seed(cfg: int, idx: int) -> int:
    return 0xD17A0000 + 16 * cfg + idx


@dataclass(frozen=True)
class Workload:
    key: str
    cfg: int
    description: str
    tensors: tuple
    launches: tuple

    def tensor(self, name: str) -> Tensor:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)

    def seed(self, name: str) -> int:
        for i, t in enumerate(self.tensors):
            if t.name == name:
                return _seed(self.cfg, i)
        raise KeyError(name)

    def algorithmic_bytes(self) -> int:
        return sum(l.algorithmic_bytes() for l in self.launches)

    def rows(self) -> int:
        return sum(l.rows for l in self.launches)


WORKLOADS = {
    "ln_1x256x1024": Workload(
        "ln_1x256x1024", 1,
        "LayerNorm (no affine, eps 1e-6) + modulate, x (1,256,1024) ~N(0,1), "
        "scale/shift (1,1024) ~N(0,0.1)",
        (Tensor("x", (256, 1024), 0.0, 1.0), Tensor("scale", (1, 1024), 0.0, 0.1),
         Tensor("shift", (1, 1024), 0.0, 0.1)),
        (Launch("ln_modulate", "ln_modulate", 256, 1024, ("x", "scale", "shift"), 1e-6),),
    ),
    "flux_1x4608x3072": Workload(
        "flux_1x4608x3072", 2,
        "FLUX.1-like adaLN (1,4608,3072): LN (no affine, eps 1e-6) + modulate on "
        "x ~N(0,1.5); gated site h = residual + gate*update, residual ~N(0,1), "
        "gate/scale/shift (1,3072) ~N(0,0.1)",
        (Tensor("x", (4608, 3072), 0.0, 1.5), Tensor("scale", (1, 3072), 0.0, 0.1),
         Tensor("shift", (1, 3072), 0.0, 0.1), Tensor("update", (4608, 3072), 0.0, 1.5),
         Tensor("residual", (4608, 3072), 0.0, 1.0), Tensor("gate", (1, 3072), 0.0, 0.1)),
        (Launch("ln_modulate", "ln_modulate", 4608, 3072, ("x", "scale", "shift"), 1e-6),
         Launch("gated_ln_modulate", "gated_ln_modulate", 4608, 3072,
                ("update", "residual", "gate", "scale", "shift"), 1e-6)),
    ),
    "ernie_1x4216x4096": Workload(
        "ernie_1x4216x4096", 3,
        "ERNIE-Image-like (1,4216,4096): weighted RMSNorm (w ~N(1,0.05), eps 1e-6) + "
        "modulate on x ~N(0,1); second site gated (update ~N(0,1), residual ~N(0,1), "
        "gate ~N(0,0.1)); scale/shift (1,4096) ~N(0,0.1)",
        (Tensor("x", (4216, 4096), 0.0, 1.0), Tensor("weight", (4096,), 1.0, 0.05),
         Tensor("scale", (1, 4096), 0.0, 0.1), Tensor("shift", (1, 4096), 0.0, 0.1),
         Tensor("update", (4216, 4096), 0.0, 1.0), Tensor("residual", (4216, 4096), 0.0, 1.0),
         Tensor("gate", (1, 4096), 0.0, 0.1)),
        (Launch("rms_modulate", "rms_modulate", 4216, 4096, ("x", "weight", "scale", "shift"),
                1e-6),
         Launch("gated_rms_modulate", "rms_modulate", 4216, 4096,
                ("update", "weight", "scale", "shift", "residual", "gate"), 1e-6,
                extra={"gated": True})),
    ),
    "glm_1x4096": Workload(
        "glm_1x4096", 4,
        "GLM-Image-like: q, k (1,4096,32,128) ~N(0,2) per-head LN(128) eps 1e-5 in one "
        "launch; hidden (1,4096,4096) ~N(0,1) LN + modulate, scale/shift ~N(0,0.1)",
        (Tensor("q", (4096 * 32, 128), 0.0, 2.0), Tensor("k", (4096 * 32, 128), 0.0, 2.0),
         Tensor("x", (4096, 4096), 0.0, 1.0), Tensor("scale", (1, 4096), 0.0, 0.1),
         Tensor("shift", (1, 4096), 0.0, 0.1)),
        (Launch("qk_layernorm", "qk_layernorm", 2 * 4096 * 32, 128, ("q", "k"), 1e-5),
         Launch("ln_modulate", "ln_modulate", 4096, 4096, ("x", "scale", "shift"), 1e-6)),
    ),
    "wan_1x96x4x480x832": Workload(
        "wan_1x96x4x480x832", 5,
        "Wan-VAE-like channels_last x [1,96,4,480,832] ~N(0,1): conv bias (96) fp32 "
        "~N(0,0.05) folded in, RMSNorm over C (gamma ~N(1,0.05), eps 1e-6) + SiLU",
        (Tensor("x", (4 * 480 * 832, 96), 0.0, 1.0), Tensor("bias", (96,), 0.0, 0.05, "f32"),
         Tensor("gamma", (96,), 1.0, 0.05, "f32_bf16vals")),
        (Launch("rmsnorm_silu_bias", "rmsnorm_silu_bias", 4 * 480 * 832, 96,
                ("x", "bias", "gamma"), 1e-6),),
    ),
    "wan_1x384x4x240x416": Workload(
        "wan_1x384x4x240x416", 6,
        "Wan-VAE-like channels_last x [1,384,4,240,416] ~N(0,1), bias/gamma (384)",
        (Tensor("x", (4 * 240 * 416, 384), 0.0, 1.0), Tensor("bias", (384,), 0.0, 0.05, "f32"),
         Tensor("gamma", (384,), 1.0, 0.05, "f32_bf16vals")),
        (Launch("rmsnorm_silu_bias", "rmsnorm_silu_bias", 4 * 240 * 416, 384,
                ("x", "bias", "gamma"), 1e-6),),
    ),
    "flux_folded_1x4608x3072": Workload(
        "flux_folded_1x4608x3072", 10,
        "FLUX.1-like LN with the modulate folded into its affine (lossy form), (1,4608,3072): "
        "x ~N(0,1.5), scale/shift (1,3072) ~N(0,0.1)",
        (Tensor("x", (4608, 3072), 0.0, 1.5), Tensor("scale", (1, 3072), 0.0, 0.1),
         Tensor("shift", (1, 3072), 0.0, 0.1)),
        (Launch("ln_modulate_folded", "ln_modulate_folded", 4608, 3072, ("x", "scale", "shift"),
                1e-6),),
    ),
    "qwen_bwd_1x6889x3072": Workload(
        "qwen_bwd_1x6889x3072", 11,
        "Qwen-Image-like final adaLN output backward, (1,6889,3072): x ~N(0,1.5), "
        "d_out ~N(0,1), scale (1,3072) ~N(0,0.1); d_x, and d_scale/d_shift by the fixed "
        "32-way fp32 token trees",
        (Tensor("x", (6889, 3072), 0.0, 1.5), Tensor("d_out", (6889, 3072), 0.0, 1.0),
         Tensor("scale", (1, 3072), 0.0, 0.1)),
        (Launch("ln_modulate_backward", "ln_modulate_backward", 6889, 3072,
                ("x", "scale", "d_out"), 1e-6, n_mod_rows=1, extra={"rows_per_batch": 6889}),),
    ),
    "qwen_bwd_2048x3x3072": Workload(
        "qwen_bwd_2048x3x3072", 12,
        "Qwen-Image-like final adaLN output backward at a large conditioning batch, "
        "(2048,3,3072): x ~N(0,1.5), d_out ~N(0,1), scale (2048,3072) ~N(0,0.1)",
        (Tensor("x", (2048 * 3, 3072), 0.0, 1.5), Tensor("d_out", (2048 * 3, 3072), 0.0, 1.0),
         Tensor("scale", (2048, 3072), 0.0, 0.1)),
        (Launch("ln_modulate_backward", "ln_modulate_backward", 2048 * 3, 3072,
                ("x", "scale", "d_out"), 1e-6, n_mod_rows=2048, extra={"rows_per_batch": 3}),),
    ),
    "flux_elementwise_1x4608x3072": Workload(
        "flux_elementwise_1x4608x3072", 7,
        "FLUX.1-like standalone modulate and residual-gate add on (1,4608,3072), bf16 and "
        "fp16 storage: x ~N(0,1.5), residual ~N(0,1), scale/shift/gate (1,3072) ~N(0,0.1)",
        (Tensor("x", (4608, 3072), 0.0, 1.5), Tensor("residual", (4608, 3072), 0.0, 1.0),
         Tensor("scale", (1, 3072), 0.0, 0.1), Tensor("shift", (1, 3072), 0.0, 0.1),
         Tensor("gate", (1, 3072), 0.0, 0.1),
         Tensor("x16", (4608, 3072), 0.0, 1.5, "f16"),
         Tensor("residual16", (4608, 3072), 0.0, 1.0, "f16"),
         Tensor("scale16", (1, 3072), 0.0, 0.1, "f16"), Tensor("shift16", (1, 3072), 0.0, 0.1, "f16"),
         Tensor("gate16", (1, 3072), 0.0, 0.1, "f16")),
        (Launch("modulate_bf16", "modulate_scale_shift", 4608, 3072, ("x", "scale", "shift"), 0.0,
                extra={"dtype": "bf16"}),
         Launch("gate_add_bf16", "residual_gate_add", 4608, 3072, ("x", "residual", "gate"), 0.0,
                extra={"dtype": "bf16"}),
         Launch("modulate_f16", "modulate_scale_shift", 4608, 3072, ("x16", "scale16", "shift16"),
                0.0, extra={"dtype": "f16"}),
         Launch("gate_add_f16", "residual_gate_add", 4608, 3072, ("x16", "residual16", "gate16"),
                0.0, extra={"dtype": "f16"})),
    ),
    "wan_epilogue_1x96x4x480x832": Workload(
        "wan_epilogue_1x96x4x480x832", 8,
        "Wan-VAE-like conv-bias epilogue with residual, channels_last [1,96,4,480,832]: "
        "x, h ~N(0,1) in bf16 and (separately drawn) fp16, bias (96) fp32 ~N(0,0.05)",
        (Tensor("x", (4 * 480 * 832, 96), 0.0, 1.0), Tensor("bias", (96,), 0.0, 0.05, "f32"),
         Tensor("h", (4 * 480 * 832, 96), 0.0, 1.0),
         Tensor("x16", (4 * 480 * 832, 96), 0.0, 1.0, "f16"),
         Tensor("h16", (4 * 480 * 832, 96), 0.0, 1.0, "f16")),
        (Launch("conv_bias_epilogue", "conv_bias_epilogue", 4 * 480 * 832, 96,
                ("x", "bias", "h"), 0.0, extra={"residual": True}),
         Launch("conv_bias_epilogue_f16", "conv_bias_epilogue", 4 * 480 * 832, 96,
                ("x16", "bias", "h16"), 0.0, extra={"residual": True, "dtype": "f16"})),
    ),
    "wan_epilogue_1x384x4x240x416": Workload(
        "wan_epilogue_1x384x4x240x416", 9,
        "Wan-VAE-like conv-bias epilogue with residual, channels_last [1,384,4,240,416]: "
        "x, h ~N(0,1) in bf16 and (separately drawn) fp16, bias (384) fp32 ~N(0,0.05)",
        (Tensor("x", (4 * 240 * 416, 384), 0.0, 1.0), Tensor("bias", (384,), 0.0, 0.05, "f32"),
         Tensor("h", (4 * 240 * 416, 384), 0.0, 1.0),
         Tensor("x16", (4 * 240 * 416, 384), 0.0, 1.0, "f16"),
         Tensor("h16", (4 * 240 * 416, 384), 0.0, 1.0, "f16")),
        (Launch("conv_bias_epilogue", "conv_bias_epilogue", 4 * 240 * 416, 384,
                ("x", "bias", "h"), 0.0, extra={"residual": True}),
         Launch("conv_bias_epilogue_f16", "conv_bias_epilogue", 4 * 240 * 416, 384,
                ("x16", "bias", "h16"), 0.0, extra={"residual": True, "dtype": "f16"})),
    ),
}


WORKLOADS["qwen_bwd_f32_2048x3x3072"] = Workload(
    "qwen_bwd_f32_2048x3x3072", 15,
    "Qwen-Image-like final adaLN output backward, the fp32 stream at a large conditioning "
    "batch, (2048,3,3072) fp32: x ~N(0,1.5), d_out ~N(0,1), scale (2048,3072) ~N(0,0.1)",
    (Tensor("x", (2048 * 3, 3072), 0.0, 1.5, "f32"), Tensor("d_out", (2048 * 3, 3072), 0.0, 1.0, "f32"),
     Tensor("scale", (2048, 3072), 0.0, 0.1, "f32")),
    (Launch("ln_modulate_backward_f32", "ln_modulate_backward", 2048 * 3, 3072,
            ("x", "scale", "d_out"), 1e-6, n_mod_rows=2048,
            extra={"rows_per_batch": 3, "dtype": "f32"}),),
)


def _flux_micro(L: int, cfg: int) -> Workload:
    """The FLUX.1 page's micro-benchmark shapes (1, L, 3072) ("[diffusion] FLUX.1
    fused adaLN modulate (bit-exact) + RoPE cache hoist, LN-affine folding
    behind quality=high", Speed Tests): the modulate chain alone, the LayerNorm
    with the fused modulate (here one lossless launch), and the folded LN."""
    key = f"flux_1x{L}x3072"
    return Workload(
        key, cfg,
        f"FLUX.1 micro-benchmark shape (1,{L},3072): x ~N(0,1.5), scale/shift (1,3072) "
        "~N(0,0.1); the modulate chain alone, LN + fused modulate, and the folded LN",
        (Tensor("x", (L, 3072), 0.0, 1.5), Tensor("scale", (1, 3072), 0.0, 0.1),
         Tensor("shift", (1, 3072), 0.0, 0.1)),
        (Launch("modulate_bf16", "modulate_scale_shift", L, 3072, ("x", "scale", "shift"), 0.0,
                extra={"dtype": "bf16"}),
         Launch("ln_modulate", "ln_modulate", L, 3072, ("x", "scale", "shift"), 1e-6),
         Launch("ln_modulate_folded", "ln_modulate_folded", L, 3072, ("x", "scale", "shift"),
                1e-6)),
    )


WORKLOADS["flux_1x4096x3072"] = _flux_micro(4096, 13)
WORKLOADS["flux_1x512x3072"] = _flux_micro(512, 14)

# The workload the headline metric is quoted on (FLUX.1-like adaLN).
HEADLINE = "flux_1x4608x3072"
