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
//  * LDS tiles are 64 x 64 bf16 with 128-byte rows and the 16-byte-chunk XOR swizzle
//    chunk ^ ((row ^ row >> 3) & 7); transposed copies ([d][row]) are built from the
//    same global loads with byte permutes.
//  * The backward pass is two kernels -- dK/dV over key tiles and dQ over query
//    tiles -- each writing its outputs once: no atomics, deterministic.
#include "kernels.h"

namespace gpt2 {
namespace {

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

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
// element offset of the 16-byte chunk `chunk` of row r in a 64-wide swizzled tile
__device__ __forceinline__ int pos(int r, int chunk) { return r * 64 + ((chunk ^ swz(r)) << 3); }
// A-row rho (0..31) of a score tile -> tile row 16(j/2) + 8g + 4(j%2) + t, rho = 8j + 4g + t
__device__ __forceinline__ int perm32(int rho) {
    const int j = rho >> 3, g = (rho >> 2) & 1, t = rho & 3;
    return 16 * (j >> 1) + 8 * g + 4 * (j & 1) + t;
}

// A 64-row x 64-column bf16 tile of a strided matrix staged through registers:
// thread t owns rows 4(t/16)..+3 and columns 4(t%16)..+3 (four 8-byte loads, rows
// >= T read as zero).  store_n writes the tile as [row][col], store_t as [col][row].
struct Tile64 {
    uint2 v[4];
    __device__ __forceinline__ void load(const bf16* g, int64_t ld, int r0, int T, int tid) {
        const int cb = tid & 15, rq = tid >> 4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = r0 + 4 * rq + rr;
            v[rr] = row < T ? *(const uint2*)(g + (int64_t)row * ld + 4 * cb) : uint2{0u, 0u};
        }
    }
    __device__ __forceinline__ void store_n(bf16* ln, int tid) const {
        const int cb = tid & 15, rq = tid >> 4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) *(uint2*)(ln + pos(4 * rq + rr, cb >> 1) + (cb & 1) * 4) = v[rr];
    }
    __device__ __forceinline__ void store_t(bf16* lt, int tid) const {
        const int cb = tid & 15, rq = tid >> 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t w0 = (j >> 1) ? v[0].y : v[0].x, w1 = (j >> 1) ? v[1].y : v[1].x;
            const uint32_t w2 = (j >> 1) ? v[2].y : v[2].x, w3 = (j >> 1) ? v[3].y : v[3].x;
            uint2 o;
            o.x = __builtin_amdgcn_perm(w1, w0, sel);
            o.y = __builtin_amdgcn_perm(w3, w2, sel);
            *(uint2*)(lt + pos(4 * cb + j, rq >> 1) + (rq & 1) * 4) = o;
        }
    }
};

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

}  // namespace

// ============================================================================ forward
// Block: 128 queries (4 waves x 32), key tiles of 64 staged in LDS.
__global__ __launch_bounds__(256) void attn_fwd_mfma64(bf16* out, float* lse, const bf16* qkv, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sbuf[2][2 * 64 * 64];  // [stage][K | V^T]
    const int nqt = (T + 127) / 128;
    const int qt = nqt - 1 - (int)blockIdx.x;  // longest rows first
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const int q0 = qt * 128, qw = q0 + 32 * w, myq = qw + r32;
    const float c = 0.125f * LOG2E;  // 1/sqrt(64) in log2 units

    u32x4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = row_frag(Qg, C3, myq, 16 * ks + 8 * g, T);
    f32x16 o[2] = {zero16(), zero16()};
    float m = -INFINITY, l = 0.f;

    const int kend = min(T, q0 + 128);
    Tile64 tk, tv;
    tk.load(Kg, C3, 0, T, tid);
    tv.load(Vg, C3, 0, T, tid);
    tk.store_n(sbuf[0], tid);
    tv.store_t(sbuf[0] + 64 * 64, tid);
    __syncthreads();
    for (int k0 = 0, it = 0; k0 < kend; k0 += 64, ++it) {
        const bf16* sK = sbuf[it & 1];
        const bf16* sVt = sK + 64 * 64;
        const bool more = k0 + 64 < kend;
        if (more) {  // next tile in flight while this one is used
            tk.load(Kg, C3, k0 + 64, T, tid);
            tv.load(Vg, C3, k0 + 64, T, tid);
        }
        if (qw < T && k0 <= qw + 31) {  // some key of this tile is visible to this wave
        const bool edge = (k0 + 63 > qw) || (k0 + 64 > T);
        float x[32];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (k0 + 32 * st > qw + 31) {  // sub-tile entirely in this wave's future
#pragma unroll
                for (int i = 0; i < 16; ++i) x[16 * st + i] = -INFINITY;
                continue;
            }
            const int kr = 32 * st + perm32(r32);
            f32x16 s = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s = mfma32(ld16(sK + pos(kr, 2 * ks + g)), qf[ks], s);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float v = s[i] * c;
                const int key = k0 + 32 * st + 16 * (i >> 3) + 8 * g + (i & 7);
                if (edge && (key > myq || key >= T)) v = -INFINITY;
                x[16 * st + i] = v;
            }
        }
        float mt = x[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mt = fmaxf(mt, x[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m, mt);
        if (__any(mn > m)) {  // rescale only when some running maximum grew
            const float corr = fast_exp2(m - mn);
            l *= corr;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                o[0][i] *= corr;
                o[1][i] *= corr;
            }
        }
        m = mn;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            if (k0 + 16 * s4 > qw + 31) break;  // remaining slices are all masked for this wave
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(x[8 * s4 + e] - mn);
                l += p[e];
            }
            const u32x4 pk = pack16<bf16>(p);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) o[dt] = mfma32(ld16(sVt + pos(32 * dt + r32, 2 * s4 + g)), pk, o[dt]);
        }
        }
        if (more) {
            tk.store_n(sbuf[(it + 1) & 1], tid);
            tv.store_t(sbuf[(it + 1) & 1] + 64 * 64, tid);
        }
        __syncthreads();
    }
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
}

// ============================================================================ backward
// D[b, h, q] = sum_d dO[q, d] O[q, d]  (= sum_k P[q, k] dP[q, k])
__global__ __launch_bounds__(256) void attn_bwd_dsum64(float* dsum, const bf16* dout, const bf16* out, int BT, int T,
                                                       int C, int NH) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, head)
    if (i >= (int64_t)BT * NH) return;
    const int row = (int)(i / NH), h = (int)(i % NH);
    const bf16* a = dout + (int64_t)row * C + h * HS;
    const bf16* o = out + (int64_t)row * C + h * HS;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < HS; d += 8) {
        float x[8], y[8];
        unpack16<bf16>(ld16(a + d), x);
        unpack16<bf16>(ld16(o + d), y);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
    }
    const int b = row / T, t = row % T;
    dsum[((int64_t)b * NH + h) * T + t] = acc;
}

// dK, dV for 128 keys (4 waves x 32), looping over query tiles of 64 at or after
// them.  P and dS are [query x key] tiles with the key as accumulator column;
// dV += P^T dO and dK += dS^T Q then take P^T / dS^T as A operands and dO^T / Q^T
// (transposed LDS copies) as B operands.
__global__ __launch_bounds__(256) void attn_bwd_dkdv_mfma64(bf16* dqkv, const bf16* qkv, const bf16* dout,
                                                            const float* lse, const float* dsum, int T, int C,
                                                            int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sbuf[2][4 * 64 * 64];  // [stage][Q | dO | Q^T | dO^T]
    __shared__ __attribute__((aligned(16))) float sLD[2][2][64];        // [stage][lse*log2e | D]
    const int kt = blockIdx.x;  // the first key tiles see the most queries: scheduled first
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const bf16* Gg = dout + (int64_t)b * T * C + h * HS;
    const int k0 = kt * 128, kw = k0 + 32 * w, mykey = kw + r32;
    const float c = 0.125f * LOG2E;

    u32x4 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        kf[ks] = row_frag(Kg, C3, mykey, 16 * ks + 8 * g, T);
        vf[ks] = row_frag(Vg, C3, mykey, 16 * ks + 8 * g, T);
    }
    f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};

    Tile64 tq, tg;
    float ld_l = 0.f, ld_d = 0.f;
    auto load_q = [&](int q0) {
        tq.load(Qg, C3, q0, T, tid);
        tg.load(Gg, C, q0, T, tid);
        if (tid < 64) {
            const int q = q0 + tid;
            ld_l = q < T ? lse[(int64_t)bh * T + q] * LOG2E : 0.f;
            ld_d = q < T ? dsum[(int64_t)bh * T + q] : 0.f;
        }
    };
    auto store_q = [&](int st) {
        bf16* b4 = sbuf[st];
        tq.store_n(b4, tid);
        tg.store_n(b4 + 64 * 64, tid);
        tq.store_t(b4 + 2 * 64 * 64, tid);
        tg.store_t(b4 + 3 * 64 * 64, tid);
        if (tid < 64) {
            sLD[st][0][tid] = ld_l;
            sLD[st][1][tid] = ld_d;
        }
    };
    if (k0 < T) {
        load_q(k0);
        store_q(0);
    }
    __syncthreads();
    for (int q0 = k0, it = 0; q0 < T; q0 += 64, ++it) {
        const bf16* sQ = sbuf[it & 1];
        const bf16* sG = sQ + 64 * 64;
        const bf16* sQt = sQ + 2 * 64 * 64;
        const bf16* sGt = sQ + 3 * 64 * 64;
        const float* sL = sLD[it & 1][0];
        const float* sD = sLD[it & 1][1];
        const bool more = q0 + 64 < T;
        if (more) load_q(q0 + 64);
        if (kw < T && q0 + 63 >= kw) {  // some query of the tile sees this wave's keys
        const bool edge = (q0 < kw + 31) || (q0 + 64 > T);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            if (q0 + 32 * qs + 31 < kw) continue;  // sub-tile entirely before this wave's keys
            const int qr = 32 * qs + perm32(r32);
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                s = mfma32(ld16(sQ + pos(qr, 2 * ks + g)), kf[ks], s);
                dp = mfma32(ld16(sG + pos(qr, 2 * ks + g)), vf[ks], dp);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                float p[8], ds[8];
                const int qlb = 32 * qs + 16 * sl + 8 * g;  // tile-local first query of this lane's 8
                const float4 l0 = *(const float4*)&sL[qlb], l1 = *(const float4*)&sL[qlb + 4];
                const float4 d0 = *(const float4*)&sD[qlb], d1 = *(const float4*)&sD[qlb + 4];
                const float Lq[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float Dq[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int q = q0 + qlb + e;
                    float pv = fast_exp2(s[8 * sl + e] * c - Lq[e]);
                    if (edge && (q >= T || mykey > q)) pv = 0.f;
                    p[e] = pv;
                    ds[e] = pv * (dp[8 * sl + e] - Dq[e]);
                }
                const u32x4 pp = pack16<bf16>(p), dd = pack16<bf16>(ds);
                const int ch = 4 * qs + 2 * sl + g;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) {
                    dv[dt] = mfma32(pp, ld16(sGt + pos(32 * dt + r32, ch)), dv[dt]);
                    dk[dt] = mfma32(dd, ld16(sQt + pos(32 * dt + r32, ch)), dk[dt]);
                }
            }
        }
        }
        if (more) store_q((it + 1) & 1);
        __syncthreads();
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
// diagonal: S^T and dP^T as in the forward pass, dS (query x 8 keys per lane) as the
// A operand of dQ = dS K with K^T from LDS.
__global__ __launch_bounds__(256) void attn_bwd_dq_mfma64(bf16* dqkv, const bf16* qkv, const bf16* dout,
                                                          const float* lse, const float* dsum, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sbuf[2][3 * 64 * 64];  // [stage][K | V | K^T]
    const int nqt = (T + 127) / 128;
    const int qt = nqt - 1 - (int)blockIdx.x;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r32 = lane & 31, g = lane >> 5;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const bf16* Gg = dout + (int64_t)b * T * C + h * HS;
    const int q0 = qt * 128, qw = q0 + 32 * w, myq = qw + r32;
    const float c = 0.125f * LOG2E;

    u32x4 qf[4], gf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qf[ks] = row_frag(Qg, C3, myq, 16 * ks + 8 * g, T);
        gf[ks] = row_frag(Gg, C, myq, 16 * ks + 8 * g, T);
    }
    const float L2 = (myq < T) ? lse[(int64_t)bh * T + myq] * LOG2E : 0.f;
    const float Dq = (myq < T) ? dsum[(int64_t)bh * T + myq] : 0.f;
    f32x16 dq[2] = {zero16(), zero16()};

    const int kend = min(T, q0 + 128);
    Tile64 tk, tv;
    tk.load(Kg, C3, 0, T, tid);
    tv.load(Vg, C3, 0, T, tid);
    tk.store_n(sbuf[0], tid);
    tv.store_n(sbuf[0] + 64 * 64, tid);
    tk.store_t(sbuf[0] + 2 * 64 * 64, tid);
    __syncthreads();
    for (int k0 = 0, it = 0; k0 < kend; k0 += 64, ++it) {
        const bf16* sK = sbuf[it & 1];
        const bf16* sV = sK + 64 * 64;
        const bf16* sKt = sK + 2 * 64 * 64;
        const bool more = k0 + 64 < kend;
        if (more) {
            tk.load(Kg, C3, k0 + 64, T, tid);
            tv.load(Vg, C3, k0 + 64, T, tid);
        }
        if (qw < T && k0 <= qw + 31) {
        const bool edge = (k0 + 63 > qw) || (k0 + 64 > T);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (k0 + 32 * st > qw + 31) continue;
            const int kr = 32 * st + perm32(r32);
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                s = mfma32(ld16(sK + pos(kr, 2 * ks + g)), qf[ks], s);
                dp = mfma32(ld16(sV + pos(kr, 2 * ks + g)), gf[ks], dp);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                float ds[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = k0 + 32 * st + 16 * sl + 8 * g + e;
                    float pv = fast_exp2(s[8 * sl + e] * c - L2);
                    if (edge && (key > myq || key >= T)) pv = 0.f;
                    ds[e] = pv * (dp[8 * sl + e] - Dq);
                }
                const u32x4 dd = pack16<bf16>(ds);
                const int ch = 4 * st + 2 * sl + g;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt) dq[dt] = mfma32(dd, ld16(sKt + pos(32 * dt + r32, ch)), dq[dt]);
            }
        }
        }
        if (more) {
            bf16* nb = sbuf[(it + 1) & 1];
            tk.store_n(nb, tid);
            tv.store_n(nb + 64 * 64, tid);
            tk.store_t(nb + 2 * 64 * 64, tid);
        }
        __syncthreads();
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
                                    hipStream_t s) {
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    ProfScope prof(s, "attn_fwd_mfma64", 4.0 * HS * pairs, 2.0 * B * T * NH * HS * 4 + 4.0 * B * NH * T);
    dim3 grid((T + 127) / 128, B * NH);
    hipLaunchKernelGGL(attn_fwd_mfma64, grid, dim3(256), 0, s, out, lse, qkv, T, C, NH);
    return hipGetLastError();
}

hipError_t attention_backward_mfma64(bf16* dqkv, float* dsum, const bf16* dout, const bf16* out, const bf16* qkv,
                                     const float* lse, int B, int T, int C, int NH, hipStream_t s) {
    const double pairs = (double)B * NH * T * (T + 1) / 2, io = 2.0 * B * T * NH * HS;
    {
        ProfScope prof(s, "attn_bwd_dsum64", 0, 2 * io + 4.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dsum64, dim3((B * T * NH + 255) / 256), dim3(256), 0, s, dsum, dout, out, B * T,
                           T, C, NH);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dkdv_mfma64", 4.0 * HS * pairs, 6 * io + 8.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dkdv_mfma64, dim3((T + 127) / 128, B * NH), dim3(256), 0, s, dqkv, qkv, dout, lse,
                           dsum, T, C, NH);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dq_mfma64", 4.0 * HS * pairs, 5 * io + 8.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dq_mfma64, dim3((T + 127) / 128, B * NH), dim3(256), 0, s, dqkv, qkv, dout, lse,
                           dsum, T, C, NH);
    }
    return hipGetLastError();
}

}  // namespace gpt2
