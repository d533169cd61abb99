// Host-side launchers of the device kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ot {

// dtype: 0 = fp32 storage, 1 = bf16 storage. in_f32: block input rows are fp32 (1) or storage (0).
hipError_t launch_qkv(int dtype, int in_f32, const QkvArgs &a, int grid, hipStream_t s);
// Token groups of 32 per wave the QKV kernel supports for a dtype / d_model (QkvArgs::tg may be
// that or 1), and the tokens per workgroup tile for a token-group count.
int qkv_max_groups(int dtype, int d_model);
int qkv_tokens_per_tile(int tg);
constexpr int QKV_SMALL_LAUNCH = 128;   // below this many two-group tiles, one group per wave
// Chunk ranges per token tile (QkvArgs::n_split) at most, for a launch with too few tiles.
int qkv_max_split(int d_model);
constexpr int QKV_SPLIT_TARGET = 512;   // workgroups a split launch aims at (two per CU)

hipError_t launch_attn(int dtype, int d_head, int stage2, const AttnArgs &a, hipStream_t s);
// Append rows (a: forward mode, R <= 32) and Stage II of the same users (b: n_cand * R <= 32) over
// the same prefix keys (a.n_pre == b.n_pre, same K/V and seq_shift), one pass over the keys.
hipError_t launch_attn_pair(int dtype, int d_head, const AttnArgs &a, const AttnArgs &b, hipStream_t s);

// Fused post-attention kernel; tokens per workgroup tile for a dtype / d_model.
hipError_t launch_post(int dtype, int resid_f32, const PostArgs &a, int grid, hipStream_t s);
int post_tokens_per_tile(int dtype, int d_model);
// Sum of a split post launch's partial rows (PostArgs::n_split > 1) into `out`, plus row statistics.
hipError_t launch_post_reduce(const PostArgs &a, int rows, hipStream_t s);
constexpr int POST_MAX_SPLIT = 8;        // hidden-chunk ranges per token tile at most
constexpr long long POST_SPLIT_BYTES = 32ll << 20;   // partials buffer at most (fp32, POST_MAX_SPLIT copies)
// bf16 storage at d = 512, unsplit launches: the wave-pair post-attention kernel (128 tokens per
// workgroup tile, like post_kernel's).
hipError_t launch_post_pair(int resid_f32, const PostArgs &a, int grid, hipStream_t s);
int post_pair_tokens_per_tile(int d_model);
// fp32 storage at d = 512: the post-attention kernel on 16x16x4 MFMA tiles (16 tokens per wave).
hipError_t launch_post_f32w(int d_model, const PostArgs &a, int grid, hipStream_t s);
int post_f32w_tokens_per_tile();

// Tokenizer kernels: grouped linear layer (rows / output features per workgroup) and [SEP] copy.
hipError_t launch_lin(int dtype, const LinArgs &a, int grid, hipStream_t s);
int lin_rows_per_tile();
int lin_features_per_tile();
hipError_t launch_sep(int dtype, const SepArgs &a, hipStream_t s);
hipError_t launch_rank(const RankArgs &a, int batch, hipStream_t s);
constexpr int RANK_MAX_EVENTS = 8192;   // timestamps of one sample staged in LDS (64 KB)

constexpr int ATTN_WAVES = 8;                    // waves per attention workgroup
constexpr int ATTN_QBLOCK = 32 * ATTN_WAVES;     // forward-mode queries per attention workgroup
constexpr int POST_MAX_DFF = 2048; // widest FFN the fused post-attention kernel stages

}  // namespace ot
