// fa_args.hpp -- what the host passes to a kernel launch, the list of built
// kernel variants, and the launcher declarations.  Host code includes only this;
// the kernels themselves live in fa_fwd_kernel.hpp and are instantiated in the
// shard files (fa_inst_*.hip).
//
// X(T, D, BC, WAVES, CAUSAL, OUT_F32) lists 16-bit-input variants; Y(WAVES, CAUSAL)
// lists fp32-input variants (head dim 64, BC = 32).  The host table and the shard
// files expand the same lists, so a variant missing from a shard is a link error.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa355 {

// One K/V stage of a 16-bit-input kernel: a K block (BC rows of D values plus one
// 16-byte pad per row, rounded up to whole 1 KB DMA instructions) and an unpadded
// V block.
constexpr int fwd_stage_bytes(int D, int BC)
{
    return 16 * ((BC * (D / 8 + 1) + 63) / 64 * 64 + BC * (D / 8));
}

// LDS bytes of a 16-bit-input kernel: two stages.
constexpr int fwd_lds_bytes(int D, int BC)
{
    return 2 * fwd_stage_bytes(D, BC);
}

// LDS bytes of the head-dim-256 kernel with two wavefronts per SIMD: two stages of
// 64-key blocks, the P^T operands four pairs exchange (16 KB), the pairs' block
// maxima and row sums (1 KB each) and the rescale flags (two block parities x four
// pairs).
constexpr int fwd_pair_lds_bytes()
{
    return 2 * fwd_stage_bytes(256, 64) + 4 * 4 * 64 * 16 + 2 * 4 * 2 * 32 * 4 + 2 * 4 * 4;
}

// LDS bytes of the head-dim-256 kernel split by role: a ring of three stages of
// 32-key blocks, P^T operands of four groups in two buffers (16 KB), their rescale
// factors and flags, and the final row sums.
constexpr int fwd_role_lds_bytes()
{
    return 3 * fwd_stage_bytes(256, 32) + 2 * 4 * 2 * 64 * 16 + 2 * 4 * 32 * 4 + 2 * 4 * 4 + 4 * 32 * 4;
}

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, N;
    int group;         // Hq / Hkv: consecutive query heads per K/V head
    int n_qtiles;      // ceil(N / BR)
    int total_tiles;   // B * Hq * n_qtiles = grid size
    float c;           // |scale| * log2(e); FLT_MIN stands in for a zero scale
    uint32_t q_sign;   // 0x80008000 flips the sign of every 16-bit Q element
    // Split-KV launches only: each query tile's key/value blocks are cut into
    // num_splits contiguous ranges, one workgroup each; partial results land in
    // o_part [num_splits,B,Hq,N,D] and lse_part [num_splits,B,Hq,N] (fp32).
    int num_splits;
    float *o_part;
    float *lse_part;
    // Additive-bias launches only: element (b, h, i, j) of the 16-bit bias is at
    // b * bias_sb + h * bias_sh + i * bias_si + j (strides in elements, 0 = shared).
    const void *bias;
    long long bias_sb, bias_sh, bias_si;
    // 8-bit-input launches only: the output multiplier (the V descale).
    float o_scale;
};

// Backward pass: gradients of sum(O * dO) with respect to Q, K and V.
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;   // [B,Hq,N] from the forward pass (natural log, scaled units)
    float *delta;       // [B,Hq,N] workspace: D_i = dO_i . O_i
    float *dq, *dk, *dv;
    int B, Hq, Hkv, N;
    int group;          // Hq / Hkv
    int dq_rows;        // queries per dQ workgroup: 128 or 256
    int n_qtiles;       // ceil(N / dq_rows): query tiles of the dQ kernel
    int total_tiles;    // B * Hq * n_qtiles
    int n_ktiles;       // ceil(N / 128): key tiles of the dK/dV kernel
    float c;            // |scale| * log2(e), FLT_MIN for a zero scale
    float scale;        // the signed scale, applied to dQ and dK
    uint32_t q_sign;    // 0x80008000 when scale < 0 (flips Q, or K, in the scores)
};

struct BF16 {};
struct F16 {};

// Launchers: one per kernel variant, explicitly instantiated in the shard files.
template <typename T, int D, int BC, int WAVES, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream);

template <int WAVES, bool CAUSAL>
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);


// Head dim 256, 128 x 64 tiles, eight wavefronts: pairs of wavefronts share 32
// query rows (fa_fwd_pair_kernel.hpp).
template <typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd_pair(const FwdArgs &a, hipStream_t stream);
// Head dim 256, 128 x 32 tiles, eight wavefronts split by role: a score and an
// output wavefront per 32 query rows (fa_fwd_role_kernel.hpp).
template <typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch_fwd_role(const FwdArgs &a, hipStream_t stream);

// Forward with an additive bias on the scaled scores.
template <typename T, int D, int BC, int WAVES, bool CAUSAL>
hipError_t launch_fwd_bias(const FwdArgs &a, hipStream_t stream);

// Split-KV forward: the partial-result kernel, then the merge kernel.
template <typename T, int D, int BC, int WAVES, bool CAUSAL>
hipError_t launch_fwd_split(const FwdArgs &a, hipStream_t stream);

// Forward with e4m3 inputs (bf16 output), head dims 64 and 128.
template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8(const FwdArgs &a, hipStream_t stream);

// Decoding against a key/value cache: the packed-group kernel over num_splits key
// ranges, then the merge kernel (fa_decode_kernel.hpp).
struct DecodeArgs {
    const void *q, *k, *v;
    float *o_part, *lse_part;      // [S, B, Hq, Nq, D] and [S, B, Hq, Nq]
    int B, Hq, Hkv, Nq, Nk;
    int group;                     // Hq / Hkv
    int rows;                      // group * Nq <= 32
    int num_splits;
    int blocks_per_split;          // 32-key blocks per piece
    float c;                       // |scale| log2(e)
    uint32_t q_sign;               // 0x80008000 flips every 16-bit Q element
};
template <typename T, int D, bool CAUSAL>
hipError_t launch_decode(const DecodeArgs &a, const FwdArgs &merge, hipStream_t stream);

// The three backward kernels (delta, dK/dV, dQ), in order on `stream`.
template <typename T, int D, bool CAUSAL>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t stream);

}  // namespace fa355

// Head dims 64 and 128: tiles 128 x 64, 128 x 32 and 256 x 64 (each also with fp32
// output), and 64 x 64.
#define FA355_VARIANTS_D64_D128(X, T, D)                                              \
    X(T, D, 64, 4, false, false) X(T, D, 64, 4, false, true)                          \
    X(T, D, 64, 4, true, false)  X(T, D, 64, 4, true, true)                           \
    X(T, D, 32, 4, false, false) X(T, D, 32, 4, false, true)                          \
    X(T, D, 32, 4, true, false)  X(T, D, 32, 4, true, true)                           \
    X(T, D, 64, 8, false, false) X(T, D, 64, 8, false, true)                          \
    X(T, D, 64, 8, true, false)  X(T, D, 64, 8, true, true)                           \
    X(T, D, 64, 2, false, false) X(T, D, 64, 2, true, false)

// Head dim 256 (four variants each: P(T, CAUSAL, OUT_F32)): the kernel split by
// role at tile 128 x 32 (the default), and the wavefront pairs at 128 x 64.
#define FA355_ROLE_VARIANTS(P, T)                                                     \
    P(T, false, false) P(T, false, true) P(T, true, false) P(T, true, true)
#define FA355_PAIR_VARIANTS(P, T) FA355_ROLE_VARIANTS(P, T)

#define FA355_VARIANTS_F32(Y) Y(1, false) Y(1, true) Y(2, false) Y(2, true) Y(4, false) Y(4, true)

// Backward variants: Z(T, D, CAUSAL), 16-bit inputs, head dims 64 and 128.
#define FA355_BWD_VARIANTS(Z, T) Z(T, 64, false) Z(T, 64, true) Z(T, 128, false) Z(T, 128, true) \
    Z(T, 256, false) Z(T, 256, true)

// Split-KV variants: S(T, D, BC, WAVES, CAUSAL): 64-key blocks, 128-row tiles at
// head dim 64 and 256-row tiles at 128.
#define FA355_SPLIT_VARIANTS(S, T, D)                                                 \
    S(T, D, 64, (D == 64 ? 4 : 8), false) S(T, D, 64, (D == 64 ? 4 : 8), true)

// Additive-bias variants, same signature: 128-row tiles, 64-key blocks at head dim
// 64 and 32-key blocks at 128 (the bias tile shares the LDS stage with K and V).
#define FA355_BIAS_VARIANTS(S, T, D)                                                  \
    S(T, D, (D == 64 ? 64 : 32), 4, false) S(T, D, (D == 64 ? 64 : 32), 4, true)
