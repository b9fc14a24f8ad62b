// fa355.cpp -- the C ABI of libfa355: argument validation, variant choice, launch.
//
// Validation runs completely before any HIP call, so every error leaves the
// outputs untouched and can be exercised on a machine without a GPU.  A valid
// call enqueues its kernels (one, or two for the split-key paths) and allocates
// nothing.
#include "fa355.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "fa_args.hpp"

namespace {

using LaunchFn = hipError_t (*)(const fa355::FwdArgs &, hipStream_t);

struct Variant {
    int dtype;      // fa355_dtype of the inputs
    int d;
    int bc;
    int waves;
    bool causal;
    bool out_f32;
    int rows;       // query rows per workgroup
    int lds;
    LaunchFn fn;
};

#define FA355_DT_BF16 FA355_BF16
#define FA355_DT_F16 FA355_F16
#define FA355_ROW(T, D, BC, W, C, O) \
    {FA355_DT_##T, D, BC, W, C, O, 32 * W, fa355::fwd_lds_bytes(D, BC), &fa355::launch_fwd<fa355::T, D, BC, W, C, O>},
#define FA355_ROW_PAIR(T, C, O) \
    {FA355_DT_##T, 256, 64, 8, C, O, 128, fa355::fwd_pair_lds_bytes(), &fa355::launch_fwd_pair<fa355::T, C, O>},
#define FA355_ROW_ROLE(T, C, O) \
    {FA355_DT_##T, 256, 32, 8, C, O, 128, fa355::fwd_role_lds_bytes(), &fa355::launch_fwd_role<fa355::T, C, O>},
#define FA355_ROW_F32(W, C) \
    {FA355_F32, 64, 32, W, C, false, 32 * W, (32 * 65 + 32 * 64) * 4, &fa355::launch_fwd_f32<W, C>},

const Variant kVariants[] = {
    FA355_VARIANTS_D64_D128(FA355_ROW, BF16, 64)
    FA355_VARIANTS_D64_D128(FA355_ROW, BF16, 128)
    FA355_ROLE_VARIANTS(FA355_ROW_ROLE, BF16)
    FA355_PAIR_VARIANTS(FA355_ROW_PAIR, BF16)
    FA355_VARIANTS_D64_D128(FA355_ROW, F16, 64)
    FA355_VARIANTS_D64_D128(FA355_ROW, F16, 128)
    FA355_ROLE_VARIANTS(FA355_ROW_ROLE, F16)
    FA355_PAIR_VARIANTS(FA355_ROW_PAIR, F16)
    FA355_VARIANTS_F32(FA355_ROW_F32)
};

int elem_bytes(int dt) { return dt == FA355_F32 ? 4 : 2; }

// A call with no query rows (B = 0 or N = 0) has nothing to compute.  Returns
// FA355_OK for it, FA355_ERR_SHAPE for sizes no call may have (negative, or head
// counts that do not divide), and 1 for a call with work to do.
int empty_call(int B, int Hq, int Hkv, int N)
{
    if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return FA355_ERR_SHAPE;
    return (B == 0 || N == 0) ? FA355_OK : 1;
}

// The built-in tile (br, bc) for an input type, head dim and sequence length,
// chosen by measurement on MI355X (interleaved timings on one device).  From 4096
// tokens at head dim 128, 256 query rows share each 64-key block (the K/V loads and
// the per-block bookkeeping are spread over more rows: 140 us against 144 us for
// 128 x 32 on the causal B1 H32 N4096 layer); shorter sequences keep 128-row tiles,
// whose lower register use fits more wavefronts per SIMD.
void default_tile(int dt, int d, int N, bool causal, int &br, int &bc)
{
    if (dt == FA355_F32) {
        br = 32;
        bc = 32;
    } else if (d == 256) {
        // The kernel split by role (fa_fwd_role_kernel), 32-key blocks: B1 H8 N8192
        // causal, inputs x3: 282-293 against 289-303 us for the wavefront pairs at
        // 128 x 64 (interleaved, four boxes), which had replaced one wavefront per
        // 32 rows (367 us).
        br = 128;
        bc = 32;
    } else if (d == 128) {
        // 256 x 64 from N = 4096 (causal) or N = 2048 (no mask), 128 x 64 below
        // (causal N = 2048: 51.4 against 53.9 us for 128 x 32; no mask, N = 1024:
        // 24.3 against 26.2 us; no mask, N = 2048: 256 x 64 69.6 against 73.0 us).
        const bool wide = N >= 4096 || (!causal && N >= 2048);
        br = wide ? 256 : 128;
        bc = 64;
    } else if (dt == FA355_BF16) {
        // d = 64, bf16 (two wavefronts per SIMD for every tile; measured on MI355X,
        // interleaved): 256 x 64 without a mask (4-8 % ahead from N = 512 up), and
        // causal from N = 2048; 128 x 32 for shorter causal rows.
        const bool wide = !causal || N >= 2048;
        br = wide ? 256 : 128;
        bc = wide ? 64 : 32;
    } else {
        // d = 64, fp16 (four wavefronts per SIMD at 128 rows): without a mask 128 x 32
        // below N = 2048 (B16 H16 N512: 27.2 against 28.3 us for 128 x 64) and 256 x 64
        // from it (B1 H16 N8192: 288 against 307 us); causal 128 x 32 below 4096 (N512:
        // 20.9 against 21.9 us) and 128 x 64 from it (N8192: 174.4 against 175.3 us).
        if (!causal) {
            br = N >= 2048 ? 256 : 128;
            bc = N >= 2048 ? 64 : 32;
        } else {
            br = 128;
            bc = N >= 4096 ? 64 : 32;
        }
    }
}

// The largest tensor any call accepts, in elements: 2^40 (4 TiB of fp32, far beyond
// one device's memory).  Under it, byte extents -- up to 256 split partials of 4
// bytes per element, 2^50 bytes -- and the overlap tests below cannot wrap.
constexpr unsigned __int128 kMaxElems = (unsigned __int128)1 << 40;

// True if a [B, H, N, d] tensor exceeds kMaxElems (sizes already checked >= 0).
bool too_large(int B, int H, int N, int d)
{
    return (unsigned __int128)B * (unsigned)H * (unsigned)N * (unsigned)d > kMaxElems;
}

// HIP counts the work-items of each grid dimension in 32 bits: a launch of `wgs`
// workgroups of `threads` work-items along one dimension needs the product below 2^32.
bool grid_fits(int64_t wgs, int threads)
{
    return wgs >= 0 && wgs <= (int64_t)UINT32_MAX / threads;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

struct Checked {
    const Variant *var;
    fa355::FwdArgs args;
    fa355_plan plan;
};

int validate(const void *q, const void *k, const void *v, const void *o, const float *lse,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
             int in_dt, int o_dt, const fa355_tuning *tuning, Checked &out)
{
    if (!q || !k || !v || !o)
        return FA355_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0)
        return FA355_ERR_SHAPE;
    if (too_large(B, Hq, N, d > 0 ? d : 0))
        return FA355_ERR_SHAPE;

    if (in_dt != FA355_F32 && in_dt != FA355_F16 && in_dt != FA355_BF16)
        return FA355_ERR_UNSUPPORTED;
    if (!(o_dt == in_dt || (o_dt == FA355_F32 && in_dt != FA355_F32)))
        return FA355_ERR_UNSUPPORTED;
    if (in_dt == FA355_F32 ? d != 64 : (d != 64 && d != 128 && d != 256))
        return FA355_ERR_UNSUPPORTED;

    // One head must fit the kernels' 32-bit byte offsets.
    const int64_t head_bytes = (int64_t)N * d * elem_bytes(in_dt);
    if (head_bytes > INT_MAX - 65536)
        return FA355_ERR_SHAPE;
    if (!std::isfinite(scale))
        return FA355_ERR_ARG;

    if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
        reinterpret_cast<uintptr_t>(v) % 16 || reinterpret_cast<uintptr_t>(o) % 16 ||
        reinterpret_cast<uintptr_t>(lse) % 4)
        return FA355_ERR_ALIGN;

    const size_t nq = (size_t)B * Hq * N * d, nkv = (size_t)B * Hkv * N * d;
    const size_t bq = nq * elem_bytes(in_dt), bkv = nkv * elem_bytes(in_dt);
    const size_t bo = nq * elem_bytes(o_dt), bl = (size_t)B * Hq * N * sizeof(float);
    if (overlaps(o, bo, q, bq) || overlaps(o, bo, k, bkv) || overlaps(o, bo, v, bkv))
        return FA355_ERR_ARG;
    if (lse && (overlaps(lse, bl, q, bq) || overlaps(lse, bl, k, bkv) ||
                overlaps(lse, bl, v, bkv) || overlaps(lse, bl, o, bo)))
        return FA355_ERR_ARG;

    int br, bc;
    default_tile(in_dt, d, N, causal != 0, br, bc);
    if (tuning && (tuning->br != 0 || tuning->bc != 0)) {
        br = tuning->br;
        bc = tuning->bc;
    }
    const bool want_f32 = o_dt == FA355_F32 && in_dt != FA355_F32;
    const Variant *var = nullptr;
    for (const Variant &x : kVariants)
        if (x.dtype == in_dt && x.d == d && x.bc == bc && x.rows == br &&
            x.causal == (causal != 0) && x.out_f32 == want_f32) {
            var = &x;
            break;
        }
    if (!var)
        return FA355_ERR_UNSUPPORTED;

    const int64_t n_qtiles = (N + br - 1) / br;
    const int64_t tiles = (int64_t)B * Hq * n_qtiles;
    if (tiles > INT_MAX || !grid_fits(tiles, 64 * var->waves))
        return FA355_ERR_SHAPE;

    fa355::FwdArgs &a = out.args;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = const_cast<void *>(o);
    a.lse = const_cast<float *>(lse);
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.group = Hq / Hkv;
    a.n_qtiles = (int)n_qtiles;
    a.total_tiles = (int)tiles;
    // exp(x * scale) = exp2(x * scale * log2 e).  A negative scale is carried by
    // negating Q (exact), so the multiplier is never negative; a zero or
    // vanishing one is raised to the smallest normal float, which leaves every
    // score at 0 after rounding and keeps -inf masks at -inf.
    float c = (float)(std::fabs((double)scale) * 1.4426950408889634);
    if (!(c >= 1.17549435e-38f))
        c = 1.17549435e-38f;
    a.c = c;
    a.q_sign = scale < 0.0f ? 0x80008000u : 0u;
    a.num_splits = 1;
    a.o_part = nullptr;
    a.lse_part = nullptr;
    a.bias = nullptr;
    a.bias_sb = a.bias_sh = a.bias_si = 0;
    a.o_scale = 1.0f;

    out.var = var;
    out.plan.br = br;
    out.plan.bc = bc;
    out.plan.waves = var->waves;
    out.plan.grid = (int)tiles;
    out.plan.lds_bytes = var->lds;
    return FA355_OK;
}

int run(const void *q, const void *k, const void *v, void *o, float *lse,
        int B, int Hq, int Hkv, int N, int d, int causal, float scale,
        int in_dt, int o_dt, const fa355_tuning *tuning, hipStream_t stream)
{
    Checked c;
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, in_dt, o_dt,
                            tuning, c);
    if (rc != FA355_OK)
        return rc;
    static const bool log = std::getenv("FA355_LOG") != nullptr;
    if (log)
        std::fprintf(stderr, "fa355: dtype=%d out_f32=%d d=%d causal=%d br=%d bc=%d grid=%d lds=%d\n",
                     in_dt, (int)c.var->out_f32, d, causal != 0, c.plan.br, c.plan.bc,
                     c.plan.grid, c.plan.lds_bytes);
    return c.var->fn(c.args, stream) == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

struct SplitVariant {
    int dtype;
    int d;
    int bc;
    bool causal;
    LaunchFn fn;
};

#define FA355_SPLIT_ROW(T, D, BC, W, C) {FA355_DT_##T, D, BC, C, &fa355::launch_fwd_split<fa355::T, D, BC, W, C>},
const SplitVariant kSplitVariants[] = {
    FA355_SPLIT_VARIANTS(FA355_SPLIT_ROW, BF16, 64)
    FA355_SPLIT_VARIANTS(FA355_SPLIT_ROW, BF16, 128)
    FA355_SPLIT_VARIANTS(FA355_SPLIT_ROW, F16, 64)
    FA355_SPLIT_VARIANTS(FA355_SPLIT_ROW, F16, 128)
};
constexpr int kMaxSplits = 16;

int run_split(const void *q, const void *k, const void *v, void *o, float *lse, int B, int Hq,
              int Hkv, int N, int d, int causal, float scale, int dt, int num_splits,
              float *o_part, float *lse_part, hipStream_t stream)
{
    if (!o_part || !lse_part)
        return FA355_ERR_NULL;
    if (dt != FA355_F16 && dt != FA355_BF16)
        return FA355_ERR_UNSUPPORTED;
    if (num_splits < 1 || num_splits > kMaxSplits)
        return FA355_ERR_ARG;
    // The split kernels use 64-key blocks: 128-row query tiles at d = 64, 256-row
    // tiles at d = 128 (measured on MI355X, B1 H2 N16384 d128 causal, 4 splits:
    // 227 us against 244 us for 128 x 32 tiles).
    const fa355_tuning tile = {d == 64 ? 128 : 256, 64};
    Checked c;
    int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dt, dt,
                      (d == 64 || d == 128) ? &tile : nullptr, c);
    if (rc != FA355_OK)
        return rc;
    if (d != 64 && d != 128)
        return FA355_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(o_part) % 16 || reinterpret_cast<uintptr_t>(lse_part) % 4)
        return FA355_ERR_ALIGN;
    const size_t rows = (size_t)B * Hq * N;
    const size_t bp = (size_t)num_splits * rows * d * 4, bl = (size_t)num_splits * rows * 4;
    const size_t nq = rows * d * 2, nkv = (size_t)B * Hkv * N * d * 2;
    struct Span { const void *p; size_t n; };
    const Span others[] = {{q, nq}, {k, nkv}, {v, nkv}, {o, nq}, {lse, lse ? rows * 4 : 0}};
    for (const Span &x : others)
        if (overlaps(o_part, bp, x.p, x.n) || overlaps(lse_part, bl, x.p, x.n))
            return FA355_ERR_ARG;
    if (overlaps(o_part, bp, lse_part, bl))
        return FA355_ERR_ARG;
    // Partial-result launch: grid * num_splits workgroups of 64 * waves; merge launch:
    // one 256-thread workgroup per 256 / (d / 4) rows.
    if ((int64_t)c.plan.grid * num_splits > INT_MAX ||
        !grid_fits((int64_t)c.plan.grid * num_splits, 64 * c.plan.waves) ||
        !grid_fits(((int64_t)rows * (d / 4) + 255) / 256, 256))
        return FA355_ERR_SHAPE;
    const SplitVariant *var = nullptr;
    for (const SplitVariant &x : kSplitVariants)
        if (x.dtype == dt && x.d == d && x.bc == tile.bc && x.causal == (causal != 0))
            var = &x;
    if (!var)
        return FA355_ERR_UNSUPPORTED;
    c.args.num_splits = num_splits;
    c.args.o_part = o_part;
    c.args.lse_part = lse_part;
    return var->fn(c.args, stream) == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

#define FA355_BIAS_ROW(T, D, BC, W, C) {FA355_DT_##T, D, BC, C, &fa355::launch_fwd_bias<fa355::T, D, BC, W, C>},
const SplitVariant kBiasVariants[] = {
    FA355_BIAS_VARIANTS(FA355_BIAS_ROW, BF16, 64)
    FA355_BIAS_VARIANTS(FA355_BIAS_ROW, BF16, 128)
    FA355_BIAS_VARIANTS(FA355_BIAS_ROW, F16, 64)
    FA355_BIAS_VARIANTS(FA355_BIAS_ROW, F16, 128)
};

int run_bias(const void *q, const void *k, const void *v, void *o, float *lse,
             const void *bias, long long sb, long long sh, long long si,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale, int dt,
             hipStream_t stream)
{
    if (!bias)
        return FA355_ERR_NULL;
    if (dt != FA355_F16 && dt != FA355_BF16)
        return FA355_ERR_UNSUPPORTED;
    // The bias kernels use the split kernels' tiles: 128 rows, 64-key blocks at
    // d = 64, 32-key blocks at d = 128.
    const fa355_tuning tile = {128, d == 64 ? 64 : 32};
    Checked c;
    int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dt, dt,
                      (d == 64 || d == 128) ? &tile : nullptr, c);
    if (rc != FA355_OK)
        return rc;
    if (d != 64 && d != 128)
        return FA355_ERR_UNSUPPORTED;
    // Rows are read four keys (8 bytes) at a time.
    if (sb < 0 || sh < 0 || si < N)
        return FA355_ERR_ARG;
    // The bias's extent in elements, in 128 bits (strides are the caller's 64-bit
    // values): beyond the largest tensor any call accepts it is too large.
    const unsigned __int128 extent = (unsigned __int128)(B - 1) * (unsigned long long)sb +
                                     (unsigned __int128)(Hq - 1) * (unsigned long long)sh +
                                     (unsigned __int128)(N - 1) * (unsigned long long)si + N;
    if (extent > kMaxElems)
        return FA355_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(bias) % 8 || si % 4 || sh % 4 || sb % 4)
        return FA355_ERR_ALIGN;
    // One (batch, head) slice of the bias is addressed with 32-bit byte offsets.
    if (((long long)(N - 1) * si + N) * 2 > INT_MAX - 65536)
        return FA355_ERR_SHAPE;
    const long long last = (long long)(B - 1) * sb + (long long)(Hq - 1) * sh + (long long)(N - 1) * si + N;
    const size_t rows = (size_t)B * Hq * N;
    if (overlaps(bias, (size_t)last * 2, o, rows * d * 2) ||
        (lse && overlaps(bias, (size_t)last * 2, lse, rows * 4)))
        return FA355_ERR_ARG;
    const SplitVariant *var = nullptr;
    for (const SplitVariant &x : kBiasVariants)
        if (x.dtype == dt && x.d == d && x.bc == tile.bc && x.causal == (causal != 0))
            var = &x;
    if (!var)
        return FA355_ERR_UNSUPPORTED;
    c.args.bias = bias;
    c.args.bias_sb = sb;
    c.args.bias_sh = sh;
    c.args.bias_si = si;
    return var->fn(c.args, stream) == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

using BwdLaunchFn = hipError_t (*)(const fa355::BwdArgs &, hipStream_t);

struct BwdVariant {
    int dtype;
    int d;
    bool causal;
    BwdLaunchFn fn;
};

#define FA355_BWD_ROW(T, D, C) {FA355_DT_##T, D, C, &fa355::launch_bwd<fa355::T, D, C>},
const BwdVariant kBwdVariants[] = {
    FA355_BWD_VARIANTS(FA355_BWD_ROW, BF16)
    FA355_BWD_VARIANTS(FA355_BWD_ROW, F16)
};

constexpr int kBwdTile = 128;   // keys per dK/dV workgroup; queries per small dQ workgroup
constexpr int kBwdTileWide = 256;   // queries per dQ workgroup while those still fill the CUs
constexpr int kBwdCus = 256;

int run_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
            const float *lse, float *dq, float *dk, float *dv, float *delta,
            int B, int Hq, int Hkv, int N, int d, int causal, float scale, int dt,
            hipStream_t stream)
{
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta)
        return FA355_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0)
        return FA355_ERR_SHAPE;
    if (too_large(B, Hq, N, d > 0 ? d : 0))
        return FA355_ERR_SHAPE;
    if ((dt != FA355_F16 && dt != FA355_BF16) || (d != 64 && d != 128 && d != 256))
        return FA355_ERR_UNSUPPORTED;
    // One head (16-bit inputs, fp32 gradients) must fit 32-bit byte offsets.
    if ((int64_t)N * d * 4 > INT_MAX - 65536)
        return FA355_ERR_SHAPE;
    if (!std::isfinite(scale))
        return FA355_ERR_ARG;
    const void *al16[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : al16)
        if (reinterpret_cast<uintptr_t>(p) % 16)
            return FA355_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(lse) % 4 || reinterpret_cast<uintptr_t>(delta) % 4)
        return FA355_ERR_ALIGN;
    const size_t nq = (size_t)B * Hq * N * d, nkv = (size_t)B * Hkv * N * d, nr = (size_t)B * Hq * N;
    struct Span { const void *p; size_t n; };
    const Span in[] = {{q, nq * 2}, {k, nkv * 2}, {v, nkv * 2}, {o, nq * 2}, {dout, nq * 2}, {lse, nr * 4}};
    const Span out[] = {{dq, nq * 4}, {dk, nkv * 4}, {dv, nkv * 4}, {delta, nr * 4}};
    for (size_t x = 0; x < 4; ++x) {
        for (const Span &i : in)
            if (overlaps(out[x].p, out[x].n, i.p, i.n))
                return FA355_ERR_ARG;
        for (size_t y = x + 1; y < 4; ++y)
            if (overlaps(out[x].p, out[x].n, out[y].p, out[y].n))
                return FA355_ERR_ARG;
    }
    const BwdVariant *var = nullptr;
    for (const BwdVariant &x : kBwdVariants)
        if (x.dtype == dt && x.d == d && x.causal == (causal != 0))
            var = &x;
    if (!var)
        return FA355_ERR_UNSUPPORTED;
    const int64_t n_tiles = (N + kBwdTile - 1) / kBwdTile;
    if ((int64_t)B * Hq * n_tiles > INT_MAX || (int64_t)B * Hq * N > INT_MAX)
        return FA355_ERR_SHAPE;
    // delta: 256 / (d / 8) rows per 256-thread workgroup; dK/dV: one 512-thread
    // workgroup per 128 keys; dQ: up to 512 threads per query tile.
    if (!grid_fits(((int64_t)B * Hq * N * (d / 8) + 255) / 256, 256) ||
        !grid_fits((int64_t)B * Hkv * n_tiles, 512) || !grid_fits((int64_t)B * Hq * n_tiles, 512))
        return FA355_ERR_SHAPE;

    fa355::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.delta = delta;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.group = Hq / Hkv;
    // 256-query dQ workgroups share each staged K/V block over twice the queries;
    // take them while there are still at least as many workgroups as CUs (head dims
    // 64 and 128: at 256 each wavefront needs a SIMD's whole register file).
    const int64_t wide = (N + kBwdTileWide - 1) / kBwdTileWide;
    a.dq_rows = d != 256 && (int64_t)B * Hq * wide >= kBwdCus ? kBwdTileWide : kBwdTile;
    a.n_qtiles = (int)(a.dq_rows == kBwdTileWide ? wide : n_tiles);
    a.total_tiles = (int)(B * Hq * a.n_qtiles);
    a.n_ktiles = (int)n_tiles;
    float c = (float)(std::fabs((double)scale) * 1.4426950408889634);
    if (!(c >= 1.17549435e-38f))
        c = 1.17549435e-38f;
    a.c = c;
    a.scale = scale;
    a.q_sign = scale < 0.0f ? 0x80008000u : 0u;
    return var->fn(a, stream) == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

// 8-bit (e4m3) inputs, bf16 output: 128-row query tiles, 64-key blocks.
constexpr int kFp8Rows = 128;

int run_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int Hq, int Hkv, int N, int d, int causal, float scale,
            float q_descale, float k_descale, float v_descale, hipStream_t stream)
{
    if (!q || !k || !v || !o)
        return FA355_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0)
        return FA355_ERR_SHAPE;
    if (too_large(B, Hq, N, d > 0 ? d : 0))
        return FA355_ERR_SHAPE;
    if (d != 64 && d != 128)
        return FA355_ERR_UNSUPPORTED;
    if ((int64_t)N * d * 2 > INT_MAX - 65536)       // one head of o, 32-bit offsets
        return FA355_ERR_SHAPE;
    const float ds[] = {q_descale, k_descale, v_descale};
    for (float x : ds)
        if (!std::isfinite(x) || !(x > 0.0f))
            return FA355_ERR_ARG;
    if (!std::isfinite(scale))
        return FA355_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
        reinterpret_cast<uintptr_t>(v) % 16 || reinterpret_cast<uintptr_t>(o) % 16 ||
        reinterpret_cast<uintptr_t>(lse) % 4)
        return FA355_ERR_ALIGN;
    const size_t nq = (size_t)B * Hq * N * d, nkv = (size_t)B * Hkv * N * d;
    const size_t bo = nq * 2, bl = (size_t)B * Hq * N * sizeof(float);
    if (overlaps(o, bo, q, nq) || overlaps(o, bo, k, nkv) || overlaps(o, bo, v, nkv))
        return FA355_ERR_ARG;
    if (lse && (overlaps(lse, bl, q, nq) || overlaps(lse, bl, k, nkv) ||
                overlaps(lse, bl, v, nkv) || overlaps(lse, bl, o, bo)))
        return FA355_ERR_ARG;
    const int64_t n_qtiles = (N + kFp8Rows - 1) / kFp8Rows;
    const int64_t tiles = (int64_t)B * Hq * n_qtiles;
    if (tiles > INT_MAX || !grid_fits(tiles, 256))
        return FA355_ERR_SHAPE;

    fa355::FwdArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.group = Hq / Hkv;
    a.n_qtiles = (int)n_qtiles;
    a.total_tiles = (int)tiles;
    // The Q and K descales join the score multiplier (computed in double, rounded
    // once); a negative scale flips the sign bit of every Q byte (exact).
    float c = (float)(std::fabs((double)scale) * (double)q_descale * (double)k_descale *
                      1.4426950408889634);
    if (!(c >= 1.17549435e-38f))
        c = 1.17549435e-38f;
    if (!std::isfinite(c))
        return FA355_ERR_ARG;
    a.c = c;
    a.q_sign = scale < 0.0f ? 0x80808080u : 0u;
    a.num_splits = 1;
    a.o_scale = v_descale;
    hipError_t e;
    if (d == 64)
        e = causal ? fa355::launch_fwd_fp8<64, true>(a, stream) : fa355::launch_fwd_fp8<64, false>(a, stream);
    else
        e = causal ? fa355::launch_fwd_fp8<128, true>(a, stream) : fa355::launch_fwd_fp8<128, false>(a, stream);
    return e == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

constexpr int kMaxDecodeSplits = 256;

// Workspace of fa_fwd_decode_noalloc: the per-piece partial results (fp32 O, then
// lse at the next 256-byte boundary), in device memory the library owns -- one copy
// per GPU, kept until the process ends.  Every call on a GPU uses that GPU's copy.
static __device__ __align__(256) unsigned char scratch[FA355_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the GPU that `stream` runs on, looked up on the first
// call for that GPU (with it made current for the lookup) and kept.  In host code the
// array's name is only a host-side handle, never a device address.
int scratch_for_stream(hipStream_t stream, unsigned char **out)
{
    static std::mutex mu;
    static unsigned char *ptr[kMaxDevices] = {};
    hipDevice_t dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA355_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess)
            return FA355_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return FA355_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess)
            return FA355_ERR_HIP;
        if (e != hipSuccess || !p)
            return FA355_ERR_HIP;
        ptr[dev] = static_cast<unsigned char *>(p);
    }
    *out = ptr[dev];
    return FA355_OK;
}

// Bytes of the no-allocation workspace a decoding call needs: S B Hq Nq d fp32 partial
// outputs, then (256-byte aligned) S B Hq Nq fp32 partial lse values.
uint64_t decode_scratch_bytes(int B, int Hq, int Nq, int d, int S)
{
    const uint64_t rows = (uint64_t)S * (uint64_t)B * (uint64_t)Hq * (uint64_t)Nq;
    return (rows * (uint64_t)d * 4 + 255) / 256 * 256 + rows * 4;
}

// own_scratch: the partial results go to `scratch` (o_part and lse_part are ignored
// and computed here, after every check has passed).
int run_decode(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, int dt,
               int num_splits, float *o_part, float *lse_part, hipStream_t stream,
               bool own_scratch = false)
{
    if (!q || !k || !v || !o || (!own_scratch && (!o_part || !lse_part)))
        return FA355_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv != 0 || (causal && Nq > Nk))
        return FA355_ERR_SHAPE;
    if (too_large(B, Hq, Nq, d > 0 ? d : 0) || too_large(B, Hkv, Nk, d > 0 ? d : 0))
        return FA355_ERR_SHAPE;
    if ((dt != FA355_F16 && dt != FA355_BF16) || (d != 64 && d != 128))
        return FA355_ERR_UNSUPPORTED;
    // The (head, query) rows of one K/V group must fit one wavefront's 32 rows.
    const int group = Hq / Hkv;
    if ((int64_t)group * Nq > 32)
        return FA355_ERR_UNSUPPORTED;
    // One K/V head plus one block past its end in 32-bit byte offsets.
    if (((int64_t)Nk + 32) * d * 2 > INT_MAX - 65536)
        return FA355_ERR_SHAPE;
    if (!std::isfinite(scale))
        return FA355_ERR_ARG;
    if (num_splits < 1 || num_splits > kMaxDecodeSplits)
        return FA355_ERR_ARG;
    if (own_scratch && decode_scratch_bytes(B, Hq, Nq, d, num_splits) > FA355_NOALLOC_SCRATCH_BYTES)
        return FA355_ERR_SHAPE;
    const void *al16[] = {q, k, v, o, own_scratch ? nullptr : o_part};
    for (const void *p : al16)
        if (reinterpret_cast<uintptr_t>(p) % 16)
            return FA355_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(lse) % 4 || reinterpret_cast<uintptr_t>(lse_part) % 4)
        return FA355_ERR_ALIGN;
    const size_t rows = (size_t)B * Hq * Nq;
    const size_t nq = rows * d * 2, nkv = (size_t)B * Hkv * Nk * d * 2;
    const size_t bp = (size_t)num_splits * rows * d * 4, bl = (size_t)num_splits * rows * 4;
    struct Span { const void *p; size_t n; };
    const Span in[] = {{q, nq}, {k, nkv}, {v, nkv}};
    // The library's own workspace cannot overlap a caller's buffer.
    const Span out[] = {{o, nq}, {lse, lse ? rows * 4 : 0}, {o_part, own_scratch ? 0 : bp},
                        {lse_part, own_scratch ? 0 : bl}};
    for (size_t x = 0; x < 4; ++x) {
        for (const Span &i : in)
            if (overlaps(out[x].p, out[x].n, i.p, i.n))
                return FA355_ERR_ARG;
        for (size_t y = x + 1; y < 4; ++y)
            if (overlaps(out[x].p, out[x].n, out[y].p, out[y].n))
                return FA355_ERR_ARG;
    }
    // Decode launch: one 64-thread workgroup per (batch, K/V head, piece); merge: one
    // 256-thread workgroup per row along x.
    if ((int64_t)B * Hkv * num_splits > INT_MAX || (int64_t)rows > INT_MAX ||
        !grid_fits((int64_t)B * Hkv * num_splits, 64) || !grid_fits((int64_t)rows, 256))
        return FA355_ERR_SHAPE;

    // Every check has passed: now (and only now) the no-allocation path looks up its
    // workspace on the GPU the stream runs on.
    if (own_scratch) {
        unsigned char *sp = nullptr;
        if (const int e = scratch_for_stream(stream, &sp); e != FA355_OK)
            return e;
        o_part = reinterpret_cast<float *>(sp);
        lse_part = reinterpret_cast<float *>(sp + (bp + 255) / 256 * 256);
    }
    float c = (float)(std::fabs((double)scale) * 1.4426950408889634);
    if (!(c >= 1.17549435e-38f))
        c = 1.17549435e-38f;
    fa355::DecodeArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Nq = Nq;
    a.Nk = Nk;
    a.group = group;
    a.rows = group * Nq;
    a.num_splits = num_splits;
    const int n_blk = (Nk + 31) / 32;
    a.blocks_per_split = (n_blk + num_splits - 1) / num_splits;
    a.c = c;
    a.q_sign = scale < 0.0f ? 0x80008000u : 0u;
    // The merge kernel sees the queries as a [B, Hq, Nq] problem.
    fa355::FwdArgs m = {};
    m.o = o;
    m.lse = lse;
    m.B = B;
    m.Hq = Hq;
    m.Hkv = Hkv;
    m.N = Nq;
    m.num_splits = num_splits;
    m.o_part = o_part;
    m.lse_part = lse_part;
    hipError_t e;
    const bool cz = causal != 0, bf = dt == FA355_BF16;
    if (d == 64)
        e = bf ? (cz ? fa355::launch_decode<fa355::BF16, 64, true>(a, m, stream)
                     : fa355::launch_decode<fa355::BF16, 64, false>(a, m, stream))
               : (cz ? fa355::launch_decode<fa355::F16, 64, true>(a, m, stream)
                     : fa355::launch_decode<fa355::F16, 64, false>(a, m, stream));
    else
        e = bf ? (cz ? fa355::launch_decode<fa355::BF16, 128, true>(a, m, stream)
                     : fa355::launch_decode<fa355::BF16, 128, false>(a, m, stream))
               : (cz ? fa355::launch_decode<fa355::F16, 128, true>(a, m, stream)
                     : fa355::launch_decode<fa355::F16, 128, false>(a, m, stream));
    return e == hipSuccess ? FA355_OK : FA355_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           fa355_dtype dtype, hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, dtype, nullptr, stream);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
              fa355_dtype in_dtype, fa355_dtype o_dtype,
              const fa355_tuning *tuning, hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, in_dtype, o_dtype, tuning,
               stream);
}

int fa_fwd_check(const void *q, const void *k, const void *v, const void *o,
                 const float *lse, int B, int Hq, int Hkv, int N, int d, int causal,
                 float scale, fa355_dtype in_dtype, fa355_dtype o_dtype,
                 const fa355_tuning *tuning, fa355_plan *plan)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0) {
        if (e == FA355_OK && plan)
            *plan = fa355_plan{};                  // no launch
        return e;
    }
    Checked c;
    const int rc = validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, in_dtype,
                            o_dtype, tuning, c);
    if (rc == FA355_OK && plan)
        *plan = c.plan;
    return rc;
}

const char *fa_status_str(int status)
{
    switch (status) {
    case FA355_OK: return "ok";
    case FA355_ERR_NULL: return "a required pointer is NULL";
    case FA355_ERR_SHAPE: return "bad shape (negative sizes, heads < 1, Hq % Hkv != 0, or too large)";
    case FA355_ERR_UNSUPPORTED: return "unsupported head dim, dtype pair or tiling";
    case FA355_ERR_ALIGN: return "misaligned pointer (16 bytes for tensors, 4 for lse)";
    case FA355_ERR_ARG: return "bad argument (non-finite scale or overlapping buffers)";
    case FA355_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, float *dq, float *dk, float *dv, float *delta,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           fa355_dtype dtype, hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale,
                   dtype, stream);
}

int fa_fwd_split(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 fa355_dtype dtype, int num_splits, float *o_part, float *lse_part,
                 hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run_split(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, num_splits,
                     o_part, lse_part, stream);
}

int fa_fwd_bias(const void *q, const void *k, const void *v, void *o, float *lse,
                const void *bias, long long bias_stride_b, long long bias_stride_h,
                long long bias_stride_row, int B, int Hq, int Hkv, int N, int d, int causal,
                float scale, fa355_dtype dtype, hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run_bias(q, k, v, o, lse, bias, bias_stride_b, bias_stride_h, bias_stride_row, B, Hq,
                    Hkv, N, d, causal, scale, dtype, stream);
}

int fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int N, int d, int causal, float scale,
               float q_descale, float k_descale, float v_descale, hipStream_t stream)
{
    if (const int e = empty_call(B, Hq, Hkv, N); e <= 0)
        return e;
    return run_fp8(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, q_descale, k_descale,
                   v_descale, stream);
}

int fa_fwd_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                  fa355_dtype dtype, int num_splits, float *o_part, float *lse_part,
                  hipStream_t stream)
{
    if (Nk < 0)
        return FA355_ERR_SHAPE;
    if (const int e = empty_call(B, Hq, Hkv, Nq); e <= 0)
        return e;
    return run_decode(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits,
                      o_part, lse_part, stream);
}

int fa_fwd_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                          float scale, fa355_dtype dtype, int num_splits, hipStream_t stream)
{
    if (Nk < 0)
        return FA355_ERR_SHAPE;
    if (const int e = empty_call(B, Hq, Hkv, Nq); e <= 0)
        return e;
    return run_decode(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits,
                      nullptr, nullptr, stream, true);
}

int fa_version(void) { return 150; }

}  // extern "C"
