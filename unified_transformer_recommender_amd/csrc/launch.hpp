// Host-side launchers of the device kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ot {

// dtype: 0 = fp32 storage, 1 = bf16 storage. tile: 0 = 64x64, 1 = 128x128 workgroup tile.
hipError_t launch_gemm(int dtype, int tile, const GemmArgs &a, int grid, hipStream_t s);

// in_f32: input rows are fp32 (1) or storage dtype (0); output is the storage dtype.
hipError_t launch_norm(int dtype, int in_f32, const NormArgs &a, hipStream_t s);

hipError_t launch_attn(int dtype, int d_head, int stage2, const AttnArgs &a, hipStream_t s);

// Fused post-attention kernel; tokens per workgroup tile for a dtype / d_model.
hipError_t launch_post(int dtype, int resid_f32, const PostArgs &a, int grid, hipStream_t s);
int post_tokens_per_tile(int dtype, int d_model);

// Workgroup tile edge of the GEMM for a given tile selector.
inline int gemm_bm(int tile) { return tile ? 128 : 64; }
inline int gemm_bn(int tile) { return tile ? 128 : 64; }
constexpr int GEMM_BK = 32;
constexpr int ATTN_QBLOCK = 128;   // forward-mode queries per attention workgroup
constexpr int POST_MAX_DFF = 2048; // widest FFN the fused post-attention kernel stages

}  // namespace ot
