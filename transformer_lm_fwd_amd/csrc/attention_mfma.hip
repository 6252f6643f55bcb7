// Causal self-attention on MFMA for bf16 operands and head size 64 (gfx950).
//
// Same computation as the row kernels ("GPT-2 from scratch with torch", 自注意力;
// "从头搭建GPT(Andrej Karpathy) 笔记", 直觉上的self-attention and attention中为什么要做
// scaling): S = q k^T / sqrt(64), keys after the query masked, softmax per query,
// O = P V; only the per-query log-sum-exp is kept for the backward pass.
//
// MFMA v_mfma_f32_32x32x16_bf16 (wave64): lane l supplies row l % 32 of A (column
// l % 32 of B) with k values 8*(l/32)..+7 of a 16-wide slice; its 16 accumulators
// hold column l % 32, rows 8*(i/4) + 4*(l/32) + i%4.
//  * Scores are computed with the query as the accumulator column (S^T = K Q^T in
//    the forward pass and for dQ, S = Q K^T with the key as the column for dK/dV).
//    The 32 A-rows of a score tile are fed a permuted set of rows, perm32(), chosen
//    so that accumulators 8s..8s+7 of lane group g = l/32 are the 8 consecutive
//    rows 16s + 8g .. +7: exactly the B (or A) fragment of the next MFMA, whose
//    reduction runs over those rows.  Probabilities never go through LDS.
//  * K/V (forward, dQ) or Q/dO (dK/dV) tiles of 64 rows x 64 bf16 go from global
//    memory straight into LDS (buffer loads to LDS) through a ring of stages, stored
//    once as [row][d]; fragments that need the transpose ([d][row]) are read with
//    ds_read_b64_tr_b16.
//  * The backward pass is two kernels -- dK/dV over key tiles and dQ over query
//    tiles -- each writing its outputs once: no atomics, deterministic.
#include <type_traits>
#include <utility>

#include "kernels.h"
#include "lds_dma.h"
#include "mx_quant.h"

namespace gpt2 {
namespace {

// Runs tile(it, std::integral_constant<int, it % NST>{}) for it = 0 .. n-1: the loop
// is unrolled NST times so that the LDS stage of each copy is a constant (its
// fragment addresses fold into the instructions' immediate offsets).
template <int NST, class F, int... S>
__device__ __forceinline__ void stage_loop_impl(int n, F&& tile, std::integer_sequence<int, S...>) {
    int it = 0;
    for (; it + NST <= n; it += NST) (tile(it + S, std::integral_constant<int, S>{}), ...);
    ((it + S < n ? tile(it + S, std::integral_constant<int, S>{}) : void()), ...);
}
template <int NST, class F> __device__ __forceinline__ void stage_loop(int n, F&& tile) {
    stage_loop_impl<NST>(n, tile, std::make_integer_sequence<int, NST>{});
}

constexpr int HS = 64;  // head size handled here
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A-row rho (0..31) of a score tile -> tile row 16(j/2) + 8g + 4(j%2) + t, rho = 8j + 4g + t
__device__ __forceinline__ int perm32(int rho) {
    const int j = rho >> 3, g = (rho >> 2) & 1, t = rho & 3;
    return 16 * (j >> 1) + 8 * g + 4 * (j & 1) + t;
}

// 16-byte fragment of a strided row (zero past T)
__device__ __forceinline__ u32x4 row_frag(const bf16* g, int64_t ld, int row, int col, int T) {
    return row < T ? ld16(g + (int64_t)row * ld + col) : u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void store4_bf16(bf16* dst, float a, float b, float c, float d) {
    uint2 v;
    v.x = pack2_bf16(a, b);
    v.y = pack2_bf16(c, d);
    *(uint2*)dst = v;
}


// ---- LDS-DMA tiles: 64 rows x 64 bf16 (128-byte rows), row-major [row][d].
// The 16-byte chunk c of row r sits at slot c ^ fsw(r), fsw(r) = 2 (r % 4) + (r / 8) % 2.
// Row-wise fragment reads (8 lanes reading one chunk of the rows perm32 picks:
// {0..3, 8..11} + 4j + 16i) and transposed reads (16 lanes reading 32 bytes of 4
// consecutive rows) both fall on distinct banks.
__device__ __forceinline__ int fsw(int r) { return ((r & 3) << 1) | ((r >> 3) & 1); }

// Per-lane offsets of one 64 x 64 tile of a row-major matrix (row stride ld
// elements, columns col0 .. col0 + 63) loaded with 8 wave loads, 2 per wave.
struct TileDma {
    static constexpr int PW = 2;
    uint32_t voff[PW];
    int w;
    __device__ __forceinline__ TileDma(int wave, int lane, int64_t col0, int64_t ld) : w(wave) {
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const int r = (wave + 4 * j) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ fsw(r);
            voff[j] = (uint32_t)(((int64_t)r * ld + col0 + c * 8) * 2);
        }
    }
    // rows row0 .. row0 + 63 enter through the scalar offset soff (bytes)
    __device__ __forceinline__ void issue(const dsc_t& d, bf16* tile, uint32_t soff) const {
#pragma unroll
        for (int j = 0; j < PW; ++j) dma16(d, lds_addr(tile + (w + 4 * j) * 512), voff[j], soff);
    }
};

// Row-wise A fragment of a score sub-tile: A-row rho = lane % 32 is tile row
// 32 st + perm32(rho), k = 16 ks + 8 g .. +7 (d).  fsw of those rows depends on the
// lane only.
struct FragK {
    int o[4];  // byte offsets for st = 0; st = 1 adds 32 rows
    __device__ __forceinline__ FragK(int r32, int g) {
        const int r = perm32(r32), f = fsw(r);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o[ks] = r * 128 + (((2 * ks + g) ^ f) << 4);
    }
    __device__ __forceinline__ u32x4 read(const bf16* tile, int st, int ks) const {
        return *(const u32x4*)((const char*)tile + o[ks] + st * 32 * 128);
    }
};

// Transposed fragment: operand row = column n = 32 dt + lane % 32 of the tile, its
// 8 k values = tile rows 16 s + 8 (lane / 32) .. +7.  fsw of the rows a lane
// addresses depends on the lane only, so per-lane bases cover every (dt, s).
struct FragT {
    int o[2];  // byte offset of the first read for dt = 0, 1 at s = 0
    __device__ __forceinline__ FragT(int lane) {
        const int gq = lane >> 4, i = lane & 15;
        const int k = 8 * (gq >> 1) + (i >> 2), f = fsw(k);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            const int col = 32 * dt + 16 * (gq & 1) + 4 * (i & 3);
            o[dt] = k * 128 + (((col >> 3) ^ f) << 4) + ((col >> 2) & 1) * 8;
        }
    }
    __device__ __forceinline__ u32x4 read(const bf16* tile, int dt, int s) const {
        return read_tr2(tile, o[dt] + s * 16 * 128, o[dt] + s * 16 * 128 + 4 * 128);
    }
};

}  // namespace

// ============================================================================ forward
// Block: 128 queries (4 waves x 32).  Key tiles of 64 rows go from global memory
// straight into LDS (K and V, each [key][d], 8 KB) through a ring of FST stages,
// so up to FST-1 tiles are in flight while one is used; two stages (32 KB) leave
// room for four blocks per CU.  K fragments are read
// row-wise (ds_read_b128), V^T fragments with transposed reads.
constexpr int FST = 2;

// q, sc non-null: also the MX FP8 codes (row stride ldq bytes) and scales ([C / 128][rows][4])
// of the stored output, for a following MX product (C % 128 == 0).
__global__ __launch_bounds__(256) void attn_fwd_mfma64(bf16* out, float* lse, const bf16* qkv, int T, int C, int NH,
                                                       uint8_t* q, int64_t ldq, uint8_t* sc) {
    __shared__ __attribute__((aligned(1024))) bf16 sbuf[FST][2][64 * 64];  // [stage][K | V]
    const int nqt = (T + 127) / 128;
    // blocks are dispatched x-fastest: every head's longest query tile goes first
    const int qt = nqt - 1 - (int)blockIdx.y;
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const int q0 = qt * 128, qw = q0 + 32 * w, myq = qw + r32;
    const float c = 0.125f * LOG2E;  // 1/sqrt(64) in log2 units

    u32x4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = row_frag(base + h * HS, C3, myq, 16 * ks + 8 * g, T);
    f32x16 o[2] = {zero16(), zero16()};
    float m = -INFINITY, l = 0.f;  // running maximum (scaled, log2 units) and sum

    // key tiles: rows of this batch's qkv block; rows >= T read as zero
    const dsc_t dsc = make_dsc(base, (uint32_t)(T * C3 * 2));
    const TileDma tk(w, lane, C + h * HS, C3), tv(w, lane, 2 * C + h * HS, C3);
    const int kend = min(T, q0 + 128);
    const int ntiles = (kend + 63) / 64;
    const FragK fk(r32, g);
    const FragT fv(lane);
    auto issue = [&](int t, int st) {
        const uint32_t soff = (uint32_t)(64 * t * C3 * 2);
        tk.issue(dsc, sbuf[st][0], soff);
        tv.issue(dsc, sbuf[st][1], soff);
    };
#pragma unroll
    for (int s0 = 0; s0 < FST - 1; ++s0)
        if (s0 < ntiles) issue(s0, s0);
    stage_loop<FST>(ntiles, [&](int it, auto stage) {
        constexpr int cur = decltype(stage)::value;
        if (it + FST - 2 < ntiles) wait_loads<TileDma::PW * 2 * (FST - 2)>();
        else wait_loads<0>();
        __builtin_amdgcn_s_barrier();
        if (it + FST - 1 < ntiles) issue(it + FST - 1, cur == 0 ? FST - 1 : cur - 1);
        const bf16* sK = sbuf[cur][0];
        const bf16* sV = sbuf[cur][1];
        const int k0 = 64 * it;
        if (qw >= T || k0 > qw + 31) return;  // no key of this tile is visible to this wave
        const bool edge = (k0 + 63 > qw) || (k0 + 64 > T);
        float x[32];  // raw scores; -inf where masked
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (k0 + 32 * st > qw + 31) {  // sub-tile entirely in this wave's future
#pragma unroll
                for (int i = 0; i < 16; ++i) x[16 * st + i] = -INFINITY;
                continue;
            }
            f32x16 sc = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sc = mfma32(fk.read(sK, st, ks), qf[ks], sc);
#pragma unroll
            for (int i = 0; i < 16; ++i) x[16 * st + i] = sc[i];
        }
        if (edge) {  // key k0 + 8 g + idx is visible iff idx <= lim (idx a constant per element)
            const int lim = min(myq, T - 1) - k0 - 8 * g;
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (16 * (i >> 3) + (i & 7) > lim) x[i] = -INFINITY;
        }
        float mt = x[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        // The reference m moves only when a score exceeds it by more than 2^8 (and on the
        // first tile): probabilities 2^(x c - m) then stay below 256, exact enough in
        // fp32 and bf16, and the rescale of o and l is rare instead of almost every tile.
        // The result does not depend on the reference beyond rounding (o / l and
        // m + log2 l are invariant).
        const float mn = mt * c > m + 8.0f ? mt * c : m;
        if (__any(mn > m)) {
            const float corr = fast_exp2(m - mn);
            l *= corr;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o[0][i] *= corr;
                o[1][i] *= corr;
            }
        }
        m = mn;
        // row sums of the bf16 probabilities (the values P V multiplies), two per
        // v_dot2c_f32_bf16 against (1, 1)
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            if (k0 + 16 * s4 > qw + 31) break;  // remaining slices are all masked for this wave
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(x[8 * s4 + e], c, -mn));
            const u32x4 pk = pack16<bf16>(p);
            // (the words are taken out of the vector one by one: a bit cast of a vector
            // element, bit_cast(bf16x2_t, pk[j]), compiles to pk[0] for every j)
            const uint32_t wd[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x2_t two;
                __builtin_memcpy(&two, &wd[j], 4);
                l = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l, false);
            }
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) o[dt] = mfma32(fv.read(sV, dt, s4), pk, o[dt]);
        }
    });
    l += __shfl_xor(l, 32, 64);
    if (myq < T) {
        const float inv = 1.0f / l;
        bf16* y = out + ((int64_t)b * T + myq) * C + h * HS;
        // o[dt][i]: column (query) r32, row d = 32 dt + 8 (i/4) + 4 g + i%4
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                store4_bf16(y + 32 * dt + 8 * i4 + 4 * g, o[dt][4 * i4] * inv, o[dt][4 * i4 + 1] * inv,
                            o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv);
        if (g == 0) lse[(int64_t)bh * T + myq] = (m + __log2f(l)) / LOG2E;
    }
    if (q) {  // kernel-uniform
        // A 32-value block (columns 32 dt .. +31 of this head) of the lane's query row is
        // held by the lane (its 16 values) and the lane 32 apart (the other 16): the block
        // maximum of the stored (bf16-rounded) values, then the lane's codes, as
        // mx_quant8 makes them.  Every lane takes part in the exchange; rows past T store
        // nothing.
        const float inv = 1.0f / l;
        const int64_t row = (int64_t)b * T + myq, nrows = (int64_t)gridDim.x / NH * T;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            float t[16];
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                t[k] = __uint_as_float((uint32_t)f32_to_bf16_bits(o[dt][k] * inv) << 16);
                amax = fmaxf(amax, fabsf(t[k]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
            const int ex = mx_exponent(amax);
            const int col = h * HS + 32 * dt;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                int w4 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(t[4 * i4], -ex),
                                                         __builtin_amdgcn_ldexpf(t[4 * i4 + 1], -ex), 0, false);
                w4 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(t[4 * i4 + 2], -ex),
                                                     __builtin_amdgcn_ldexpf(t[4 * i4 + 3], -ex), w4, true);
                if (myq < T) *(uint32_t*)(q + row * ldq + col + 8 * i4 + 4 * g) = (uint32_t)w4;
            }
            if (g == 0 && myq < T) sc[((int64_t)(col / 128) * nrows + row) * 4 + (col % 128) / 32] = (uint8_t)(ex + 127);
        }
    }
}

// ============================================================================ backward
// The per-query values both backward kernels need -- LD[b, h, q] = {lse[q] log2 e,
// D[q]} with D[q] = sum_d dO[q, d] O[q, d] (= sum_k P[q, k] dP[q, k]) -- are
// computed by the dQ kernel, which runs first, and stored side by side so that a
// 64-query tile of them is one load for the dK/dV kernel.
constexpr int BST = 3;  // LDS stages of the backward kernels

// dK, dV for 128 keys (4 waves x 32), looping over query tiles of 64 at or after
// them.  Q and dO tiles ([q][d]) and their {L, D} values arrive by LDS DMA in a
// BST-stage ring.  P and dS are [query x key] tiles with the key as accumulator
// column (A = Q / dO rows, B = this lane's K / V row); dV += P^T dO and
// dK += dS^T Q take P^T / dS^T as A operands and dO^T / Q^T (transposed reads of
// the same tiles) as B operands.
// Register budget for three waves per SIMD (170 VGPRs; the kernel would otherwise
// take ~180 and run two).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_bwd_dkdv_mfma64(
    bf16* dqkv, const bf16* qkv, const bf16* dout, const float2* LD, int T, int C, int NH) {
    __shared__ __attribute__((aligned(1024))) bf16 sbuf[BST][2][64 * 64];  // [stage][Q | dO]
    __shared__ __attribute__((aligned(1024))) float sLD[BST][256];         // [stage][{L, D} x 64, copy]
    const int kt = blockIdx.y;  // the first key tiles see the most queries: dispatched first
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const int k0 = kt * 128, kw = k0 + 32 * w, mykey = kw + r32;
    const float c = 0.125f * LOG2E;

    u32x4 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = row_frag(base + C + h * HS, C3, mykey, 16 * ks + 8 * g, T);
        vf[ks] = row_frag(base + 2 * C + h * HS, C3, mykey, 16 * ks + 8 * g, T);
    }
    f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};

    const dsc_t dq_ = make_dsc(base, (uint32_t)(T * C3 * 2));
    const dsc_t dg = make_dsc(dout + (int64_t)b * T * C, (uint32_t)((int64_t)T * C * 2));
    const dsc_t dl = make_dsc(LD + (int64_t)bh * T, (uint32_t)(T * 8));
    const TileDma tq(w, lane, h * HS, C3), tg(w, lane, h * HS, C);
    const FragK fk(r32, g);
    const FragT ft(lane);
    const int ntiles = k0 < T ? (T - k0 + 63) / 64 : 0;
    auto issue = [&](int t, int st) {
        const int q0 = k0 + 64 * t;
        tq.issue(dq_, sbuf[st][0], (uint32_t)(q0 * C3 * 2));
        tg.issue(dg, sbuf[st][1], (uint32_t)(q0 * C * 2));
        if (w == 0) dma16(dl, lds_addr(sLD[st]), (uint32_t)((lane & 31) * 16), (uint32_t)(q0 * 8));
    };
#pragma unroll
    for (int s0 = 0; s0 < BST - 1; ++s0)
        if (s0 < ntiles) issue(s0, s0);
    int cur = 0;
    for (int it = 0; it < ntiles; ++it) {
        if (it + BST - 2 < ntiles) {
            if (w == 0) wait_loads<(2 * TileDma::PW + 1) * (BST - 2)>();
            else wait_loads<2 * TileDma::PW * (BST - 2)>();
        } else {
            wait_loads<0>();
        }
        __builtin_amdgcn_s_barrier();
        if (it + BST - 1 < ntiles) issue(it + BST - 1, cur == 0 ? BST - 1 : cur - 1);
        const bf16* sQ = sbuf[cur][0];
        const bf16* sG = sbuf[cur][1];
        const float* sL = sLD[cur];
        cur = cur + 1 == BST ? 0 : cur + 1;
        const int q0 = k0 + 64 * it;
        if (kw >= T || q0 + 63 < kw) continue;  // no query of the tile sees this wave's keys
        const bool edge = (q0 < kw + 31) || (q0 + 64 > T);
        // query q0 + 8 g + idx sees this lane's key iff lo <= idx < hi
        const int lo = mykey - q0 - 8 * g, hi = T - q0 - 8 * g;
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            if (q0 + 32 * qs + 31 < kw) continue;  // sub-tile entirely before this wave's keys
            f32x16 sc = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                sc = mfma32(fk.read(sQ, qs, ks), kf[ks], sc);
                dp = mfma32(fk.read(sG, qs, ks), vf[ks], dp);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const int qlb = 32 * qs + 16 * sl + 8 * g;  // tile-local first query of this lane's 8
                float Lq[8], Dq[8];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const float4 v = *(const float4*)&sL[2 * qlb + 4 * e4];
                    Lq[2 * e4] = v.x; Dq[2 * e4] = v.y; Lq[2 * e4 + 1] = v.z; Dq[2 * e4 + 1] = v.w;
                }
                float p[8], ds[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(sc[8 * sl + e], c, -Lq[e]));
                if (edge) {  // wave-uniform: only tiles on the diagonal or past T mask
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int idx = 32 * qs + 16 * sl + e;
                        if (idx < lo || idx >= hi) p[e] = 0.f;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ds[e] = p[e] * (dp[8 * sl + e] - Dq[e]);
                const u32x4 pp = pack16<bf16>(p), dd = pack16<bf16>(ds);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    dv[dt] = mfma32(pp, ft.read(sG, dt, 2 * qs + sl), dv[dt]);
                    dk[dt] = mfma32(dd, ft.read(sQ, dt, 2 * qs + sl), dk[dt]);
                }
            }
        }
    }
    // dv[dt][i] / dk[dt][i]: column d = 32 dt + r32, row key kw + 8 (i/4) + 4 g + i%4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = kw + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key < T) {
            bf16* row = dqkv + ((int64_t)b * T + key) * C3 + h * HS;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                row[C + 32 * dt + r32] = from_f32<bf16>(dk[dt][i] * 0.125f);
                row[2 * C + 32 * dt + r32] = from_f32<bf16>(dv[dt][i]);
            }
        }
    }
}

// dQ for 128 queries (4 waves x 32), looping over key tiles of 64 up to the
// diagonal (K and V tiles by LDS DMA, as in the forward pass): S^T and dP^T with
// the query as accumulator column, dS (query x 8 keys per lane) as the A operand
// of dQ = dS K with K^T fragments read transposed from the K tile.
__global__ __launch_bounds__(256) void attn_bwd_dq_mfma64(bf16* dqkv, const bf16* qkv, const bf16* dout,
                                                          const bf16* out, const float* lse, float2* LD, int T,
                                                          int C, int NH) {
    __shared__ __attribute__((aligned(1024))) bf16 sbuf[BST][2][64 * 64];  // [stage][K | V]
    const int nqt = (T + 127) / 128;
    const int qt = nqt - 1 - (int)blockIdx.y;  // longest first
    const int bh = blockIdx.x, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Gg = dout + (int64_t)b * T * C + h * HS;
    const int q0 = qt * 128, qw = q0 + 32 * w, myq = qw + r32;
    const float c = 0.125f * LOG2E;

    u32x4 qf[4], gf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qf[ks] = row_frag(base + h * HS, C3, myq, 16 * ks + 8 * g, T);
        gf[ks] = row_frag(Gg, C, myq, 16 * ks + 8 * g, T);
    }
    // D = sum_d dO[q, d] O[q, d]: this lane holds 32 of the 64 dims (the same as its
    // dO fragments), the lane 32 apart the other 32.  {lse log2 e, D} is stored for
    // the dK/dV kernel, which runs next.
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        float gv[8], ov[8];
        unpack16<bf16>(gf[ks], gv);
        unpack16<bf16>(row_frag(out + (int64_t)b * T * C + h * HS, C, myq, 16 * ks + 8 * g, T), ov);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart += gv[e] * ov[e];
    }
    const float Dq = dpart + __shfl_xor(dpart, 32, 64);
    const float2 ldq = make_float2(myq < T ? lse[(int64_t)bh * T + myq] * LOG2E : 0.f, Dq);
    if (g == 0 && myq < T) LD[(int64_t)bh * T + myq] = ldq;
    f32x16 dq[2] = {zero16(), zero16()};
    f32x16 negD;
#pragma unroll
    for (int i = 0; i < 16; ++i) negD[i] = -Dq;

    const dsc_t dsc = make_dsc(base, (uint32_t)(T * C3 * 2));
    const TileDma tk(w, lane, C + h * HS, C3), tv(w, lane, 2 * C + h * HS, C3);
    const FragK fk(r32, g);
    const FragT ft(lane);
    const int kend = min(T, q0 + 128);
    const int ntiles = (kend + 63) / 64;
    auto issue = [&](int t, int st) {
        const uint32_t soff = (uint32_t)(64 * t * C3 * 2);
        tk.issue(dsc, sbuf[st][0], soff);
        tv.issue(dsc, sbuf[st][1], soff);
    };
#pragma unroll
    for (int s0 = 0; s0 < BST - 1; ++s0)
        if (s0 < ntiles) issue(s0, s0);
    int cur = 0;
    for (int it = 0; it < ntiles; ++it) {
        if (it + BST - 2 < ntiles) wait_loads<2 * TileDma::PW * (BST - 2)>();
        else wait_loads<0>();
        __builtin_amdgcn_s_barrier();
        if (it + BST - 1 < ntiles) issue(it + BST - 1, cur == 0 ? BST - 1 : cur - 1);
        const bf16* sK = sbuf[cur][0];
        const bf16* sV = sbuf[cur][1];
        cur = cur + 1 == BST ? 0 : cur + 1;
        const int k0 = 64 * it;
        if (qw >= T || k0 > qw + 31) continue;
        const bool edge = (k0 + 63 > qw) || (k0 + 64 > T);
        const int lim = min(myq, T - 1) - k0 - 8 * g;  // key k0 + 8 g + idx visible iff idx <= lim
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (k0 + 32 * st > qw + 31) continue;
            // the sub-tile's fragments are all requested before its first product
            u32x4 kr[4], vr[4], kt[2][2];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kr[ks] = fk.read(sK, st, ks);
                vr[ks] = fk.read(sV, st, ks);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) kt[sl][dt] = ft.read(sK, dt, 2 * st + sl);
            // dP - D directly: the dP product starts from -D (this lane's query is the
            // accumulator column, so one register block serves every tile)
            f32x16 sc = zero16(), dp = negD;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                sc = mfma32(kr[ks], qf[ks], sc);
                dp = mfma32(vr[ks], gf[ks], dp);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                float pv[8], ds[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(sc[8 * sl + e], c, -ldq.x));
                if (edge) {  // wave-uniform
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (32 * st + 16 * sl + e > lim) pv[e] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ds[e] = pv[e] * dp[8 * sl + e];
                const u32x4 dd = pack16<bf16>(ds);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) dq[dt] = mfma32(dd, kt[sl][dt], dq[dt]);
            }
        }
    }
    // dq[dt][i]: column d = 32 dt + r32, row query qw + 8 (i/4) + 4 g + i%4
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int q = qw + 8 * (i >> 2) + 4 * g + (i & 3);
        if (q < T) {
            bf16* row = dqkv + ((int64_t)b * T + q) * C3 + h * HS;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) row[32 * dt + r32] = from_f32<bf16>(dq[dt][i] * 0.125f);
        }
    }
}

// ============================================================================ launchers
hipError_t attention_forward_mfma64(bf16* out, float* lse, const bf16* qkv, int B, int T, int C, int NH,
                                    hipStream_t s, uint8_t* q, int64_t ldq, uint8_t* sc) {
    if (q && (!sc || C % 128 || ldq < C || ldq % 16)) return hipErrorInvalidValue;
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    ProfScope prof(s, q ? "attn_fwd_mfma64_mx" : "attn_fwd_mfma64", 4.0 * HS * pairs,
                   2.0 * B * T * NH * HS * 4 + 4.0 * B * NH * T + (q ? (double)B * T * C * (1 + 1 / 32.) : 0.0));
    dim3 grid(B * NH, (T + 127) / 128);
    hipLaunchKernelGGL(attn_fwd_mfma64, grid, dim3(256), 0, s, out, lse, qkv, T, C, NH, q, ldq, sc);
    return hipGetLastError();
}

hipError_t attention_backward_mfma64(bf16* dqkv, float* dsum, const bf16* dout, const bf16* out, const bf16* qkv,
                                     const float* lse, int B, int T, int C, int NH, hipStream_t s) {
    const double pairs = (double)B * NH * T * (T + 1) / 2, io = 2.0 * B * T * NH * HS;
    {
        ProfScope prof(s, "attn_bwd_dq_mfma64", 4.0 * HS * pairs, 6 * io + 12.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dq_mfma64, dim3(B * NH, (T + 127) / 128), dim3(256), 0, s, dqkv, qkv, dout, out,
                           lse, (float2*)dsum, T, C, NH);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dkdv_mfma64", 4.0 * HS * pairs, 6 * io + 8.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dkdv_mfma64, dim3(B * NH, (T + 127) / 128), dim3(256), 0, s, dqkv, qkv, dout,
                           (const float2*)dsum, T, C, NH);
    }
    return hipGetLastError();
}

}  // namespace gpt2
