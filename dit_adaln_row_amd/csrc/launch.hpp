// Internal interface between the C-ABI layer (abi.hip) and the kernel files.
// Every launcher assumes its arguments were validated by the ABI layer:
// sizes in range, pointers 16-byte aligned, no illegal aliasing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditnorm {

struct DeviceInfo {
  int num_cu;        // compute units
  int device;        // HIP device ordinal
};

// Row kernels: LayerNorm or RMSNorm of each row + adaLN modulate, with an
// optional gated-residual stage in front.
struct RowArgs {
  const uint16_t *x;         // update (gated) or input rows, bf16 [rows, cols]
  const uint16_t *residual;  // gated only
  const uint16_t *gate;      // gated only, [B, mod_stride]
  const uint16_t *scale;     // [B, mod_stride]
  const uint16_t *shift;     // [B, mod_stride]
  const uint16_t *weight;    // RMS only, [cols]
  uint16_t *residual_out;    // gated only
  uint16_t *out;
  float *mean_out;           // optional (LN only)
  float *rstd_out;           // optional
  uint16_t *y_out;           // optional
  int64_t rows;
  int64_t rows_per_batch;
  int64_t mod_stride;
  int32_t cols;
  float eps;
  int64_t full_blocks;       // balanced kernel: workgroups of 4 whole rows (set by the launcher)
};
// fold: the affine-folded LN form (LN only: rms and gated false)
hipError_t launch_row(const RowArgs &a, bool rms, bool gated, bool fold, const DeviceInfo &dev,
                      hipStream_t stream);

// Per-head LayerNorm over 128-wide rows of q then k.
struct QkArgs {
  const uint16_t *q;
  const uint16_t *k;
  uint16_t *q_out;
  uint16_t *k_out;
  float *mean_out;  // optional [rows_q + rows_k]
  float *rstd_out;  // optional
  int64_t rows_q;
  int64_t rows_k;
  int32_t head_dim;  // a multiple of 8, at most 128
  float eps;
};
hipError_t launch_qk(const QkArgs &a, const DeviceInfo &dev, hipStream_t stream);

// channels_last [bias] + RMSNorm over C + gamma + SiLU.
struct WanArgs {
  const uint16_t *x;
  const float *bias;   // nullable
  const float *gamma;
  uint16_t *out;
  float *rstd_out;     // optional
  uint16_t *xb_out;    // optional
  int64_t rows;
  int32_t channels;
  float eps;
};
hipError_t launch_wan(const WanArgs &a, const DeviceInfo &dev, hipStream_t stream);

// channels_last conv-bias epilogue (+ residual).
// x, h, out of storage type dtype (0 bf16, 1 fp16, 2 fp32); bias of
// bias_dtype (2 fp32, else equal to dtype).
struct EpilogueArgs {
  const void *x;
  const void *bias;
  const void *h;       // nullable
  void *out;
  int64_t rows;
  int32_t channels;
  int32_t dtype;
  int32_t bias_dtype;
};
hipError_t launch_epilogue(const EpilogueArgs &a, const DeviceInfo &dev, hipStream_t stream);

// Standalone elementwise stages: op 0 modulate (a = x, m0 = scale, m1 = shift),
// op 1 residual-gate add (a = update, b = residual, m0 = gate); dtype 0 bf16,
// 1 fp16.
struct ElementwiseArgs {
  const uint16_t *a;
  const uint16_t *b;
  const uint16_t *m0;
  const uint16_t *m1;
  uint16_t *out;
  int64_t rows;
  int64_t rows_per_batch;
  int64_t mod_stride;
  int32_t cols;
};
hipError_t launch_elementwise(const ElementwiseArgs &a, int op, int dtype, const DeviceInfo &dev,
                              hipStream_t stream);

// Backward of LN (no affine) + modulate: d_x, and the token sums d_scale,
// d_shift by fixed balanced trees.
// x, scale, d_out, d_x of storage type dtype (0 bf16, 2 fp32).
struct BwdArgs {
  const void *x;          // [rows, cols]
  const void *scale;      // [B, mod_stride]
  const void *d_out;      // [rows, cols]
  void *d_x;              // [rows, cols]
  float *d_scale;         // [B, cols]
  float *d_shift;         // [B, cols]
  float *mean_out;        // optional [rows]
  float *rstd_out;        // optional [rows]
  int64_t rows;
  int64_t rows_per_batch;
  int64_t mod_stride;
  int32_t cols;
  float eps;
  int32_t dtype;
};
// Workspace layout (byte offsets; every region 256-byte aligned): the
// partial tree sums.  None when a batch has at most rows_per_chunk tokens.
struct BwdLayout {
  int rows_per_chunk;               // tokens per workgroup of the fused kernel (4 or 8)
  int64_t chunks;                   // per batch: ceil(rows_per_batch / rows_per_chunk)
  int64_t part0_off, part0_floats;  // per sum: B * chunks * cols (0 if chunks == 1)
  int64_t part1_off, part1_floats;  // per sum: B * (first tree level's count) * cols,
                                    // 0 if that level is the last
  int64_t bytes;
};
BwdLayout bwd_layout(int64_t rows, int64_t cols, int64_t rows_per_batch, int dtype);
hipError_t launch_backward(const BwdArgs &a, const BwdLayout &L, float *part0, float *part1,
                           hipStream_t stream);

// Plain 16-byte copy (measurement utility).
hipError_t launch_copy(const void *src, void *dst, int64_t bytes, const DeviceInfo &dev,
                       hipStream_t stream);

// Persistent-grid size: min(work units, CUs x resident blocks per CU).
template <typename K>
inline int64_t persistent_grid(K kernel, int block, int64_t units, const DeviceInfo &dev,
                               int min_per_cu = 1) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
      per_cu < min_per_cu)
    per_cu = min_per_cu;
  const int64_t g = (int64_t)dev.num_cu * per_cu;
  return units < g ? units : g;
}

}  // namespace ditnorm
