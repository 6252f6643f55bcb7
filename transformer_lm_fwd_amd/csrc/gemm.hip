// MFMA-tiled GEMM for gfx950 with the fused epilogues of the GPT-2 step.
//
// Every linear layer of the model is a matrix product plus a bias repeated over
// the rows ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン", ニューラルネットワーク層の実装),
// weights stored (out, in) row-major.  The step needs three operand layouts:
//   forward   Y  = X  W^T : A = X  (k-contiguous), B = W (k-contiguous)
//   dX        dX = dY W   : A = dY (k-contiguous), B = W (n-contiguous)
//   dW        dW = dY^T X : A = dY (m-contiguous), B = X (n-contiguous)
// bf16 operands go from global memory straight into LDS (buffer loads to LDS) in
// the layout they have in memory; a k-contiguous tile is read back with
// ds_read_b128 and an mn-contiguous one with the transposing ds_read_b64_tr_b16,
// so no operand is transposed in registers.  bf16 products use
// v_mfma_f32_32x32x16_bf16, fp32 products v_mfma_f32_16x16x4_f32 on tiles staged
// through registers.  The sum over k does not depend on which k values a lane
// group supplies as long as A and B agree, so both operands use the same per-lane
// k offsets.
#include <algorithm>
#include <mutex>
#include <set>
#include <string>

#include "kernels.h"
#include "lds_dma.h"
#include "mx_quant.h"

namespace gpt2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// MFMA shapes.  bf16: v_mfma_f32_32x32x16_bf16 (the 16x16x32 form issues at half
// its rate on gfx950).  Lane l supplies row l % 32 of a 32-row A block (B: column
// l % 32) with the 8 k values 8*(l/32)..+7 of a 16-wide k slice; its 16
// accumulators hold column l % 32, rows 8*(i/4) + 4*(l/32) + i%4.
// fp32: v_mfma_f32_16x16x4_f32, four per 16-byte fragment (lane l: row l % 16,
// k = 4*(l/16) + e for the e-th instruction); accumulators: column l % 16, rows
// 4*(l/16) + i.  Only the pairing of A and B k values matters for the sum, so
// both operands use the same per-lane k offsets.
template <class T> struct MfmaTraits;
template <> struct MfmaTraits<bf16> {
    static constexpr int TILE = 32, KSLICE = 16, NACC = 16;
    typedef float acc_t __attribute__((ext_vector_type(16)));
    __device__ static __forceinline__ int frag_row(int lane) { return lane & 31; }
    __device__ static __forceinline__ int frag_k(int lane) { return (lane >> 5) * 8; }
    __device__ static __forceinline__ int out_row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
    __device__ static __forceinline__ int out_col(int lane) { return lane & 31; }
    __device__ static __forceinline__ acc_t step(const u32x4& a, const u32x4& b, acc_t acc) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct MfmaTraits<float> {
    static constexpr int TILE = 16, KSLICE = 16, NACC = 4;
    typedef f32x4 acc_t;
    __device__ static __forceinline__ int frag_row(int lane) { return lane & 15; }
    __device__ static __forceinline__ int frag_k(int lane) { return (lane >> 4) * 4; }
    __device__ static __forceinline__ int out_row(int lane, int i) { return 4 * (lane >> 4) + i; }
    __device__ static __forceinline__ int out_col(int lane) { return lane & 15; }
    __device__ static __forceinline__ acc_t step(const u32x4& a, const u32x4& b, acc_t acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
        return acc;
    }
};

// Transpose a KV x KV block held as KV 16-byte rows (row r = k, element j = mn)
// into KV 16-byte rows indexed by mn holding KV consecutive k.
template <class T> __device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out);
template <> __device__ __forceinline__ void transpose_block<float>(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[j][r] = in[r][j];
}
template <> __device__ __forceinline__ void transpose_block<bf16>(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1, sh = (j & 1) * 16;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t lo = (in[2 * p][w] >> sh) & 0xffffu;
            uint32_t hi = (in[2 * p + 1][w] >> sh) & 0xffffu;
            out[j][p] = lo | (hi << 16);
        }
    }
}

// Loads one ROWS x BK tile of an operand into registers and stores it to LDS,
// k-contiguous with row pitch PITCH elements.
template <class T, bool KCONTIG, int ROWS, int BK, int NT>
struct TileLoader {
    static constexpr int KV = Vec16<T>::N;
    // k-contiguous: ROWS * BK / KV chunks of 16 bytes
    static constexpr int NCHUNK = ROWS * (BK / KV);
    // mn-contiguous: KV x KV blocks
    static constexpr int NBLK = (BK / KV) * (ROWS / KV);
    static constexpr int NREG = KCONTIG ? (NCHUNK + NT - 1) / NT : ((NBLK + NT - 1) / NT) * KV;
    u32x4 r[NREG];

    // rows: valid rows [0, nrows) of this tile; k range valid [0, kvalid)
    __device__ __forceinline__ void load(const T* base, int64_t ld, int row0, int nrows, int k0, int kend, int tid) {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < NREG; ++i) {
                int c = tid + i * NT;
                int row = c / (BK / KV), kc = c % (BK / KV);
                int k = k0 + kc * KV;
                bool ok = (c < NCHUNK) && (row0 + row < nrows) && (k < kend);
                r[i] = ok ? ld16(base + (int64_t)(row0 + row) * ld + k) : u32x4{0, 0, 0, 0};
            }
        } else {
#pragma unroll
            for (int i = 0; i < NREG / KV; ++i) {
                int b = tid + i * NT;
                int kb = b / (ROWS / KV), mb = b % (ROWS / KV);
                int mn = row0 + mb * KV;
                bool okb = (b < NBLK) && (mn < nrows);
#pragma unroll
                for (int rr = 0; rr < KV; ++rr) {
                    int k = k0 + kb * KV + rr;
                    bool ok = okb && (k < kend);
                    r[i * KV + rr] = ok ? ld16(base + (int64_t)k * ld + mn) : u32x4{0, 0, 0, 0};
                }
            }
        }
    }
    template <int PITCH>
    __device__ __forceinline__ void store(T* lds, int tid) {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < NREG; ++i) {
                int c = tid + i * NT;
                if (c < NCHUNK) {
                    int row = c / (BK / KV), kc = c % (BK / KV);
                    st16(lds + row * PITCH + kc * KV, r[i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NREG / KV; ++i) {
                int b = tid + i * NT;
                if (b < NBLK) {
                    int kb = b / (ROWS / KV), mb = b % (ROWS / KV);
                    u32x4 t[KV];
                    transpose_block<T>(&r[i * KV], t);
#pragma unroll
                    for (int j = 0; j < KV; ++j) st16(lds + (mb * KV + j) * PITCH + kb * KV, t[j]);
                }
            }
        }
    }
};

template <class T, int EPI>
__device__ __forceinline__ void epilogue_store(const GemmArgs& a, float* wsC, int row, int col, float v) {
    if (row >= a.M || col >= a.N) return;
    const int64_t o = (int64_t)row * a.ldc + col;
    if constexpr (EPI == EPI_F32) {
        wsC[o] = v;
    } else {
        T* C = (T*)a.C;
        if constexpr (EPI == EPI_BIAS) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(v);
        } else if constexpr (EPI == EPI_BIAS_RES) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(to_f32(((const T*)a.R)[o]) + v);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(v);
            ((T*)a.C2)[o] = from_f32<T>(gelu_fwd(v));
        } else if constexpr (EPI == EPI_GELU_BWD) {
            C[o] = from_f32<T>(v * gelu_bwd(to_f32(((const T*)a.R)[o])));
        }
    }
}

// Block -> output tile.  Workgroup i runs on XCD i % 8 (round-robin dispatch), and
// each XCD has its own L2.  So each XCD is given a contiguous range of tiles, and
// tiles are numbered in groups of 8 tile-rows walked column by column: the ~64
// blocks resident on one XCD then cover an 8 x 8 square of tiles and share their
// A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_order(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int q = ntiles / 8, r = ntiles % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int t = xcd * q + min(xcd, r) + idx;
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (t / per_group) * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int in = t % per_group;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

template <class T, bool AK, bool BKC, int EPI, int BM, int BN, int BK, int WM, int WN, bool ORDER = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a, int k_per_split, int64_t split_stride) {
    constexpr int NT = 64 * WM * WN;
    constexpr int KV = Vec16<T>::N;
    constexpr int PITCH = BK + KV;
    using MT = MfmaTraits<T>;
    constexpr int MTILE = MT::TILE;
    constexpr int TM = BM / WM / MTILE, TN = BN / WN / MTILE;
    constexpr int KSLICE = MT::KSLICE;
    constexpr int SA = BM * PITCH, SB = BN * PITCH;
    __shared__ __attribute__((aligned(16))) T lds[2][SA + SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm = blockIdx.y, tn = blockIdx.x;
    if constexpr (ORDER) tile_order(blockIdx.x, (a.M + BM - 1) / BM, (a.N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * k_per_split;
    const int kend = min(a.K, kbeg + k_per_split);
    const T* A = (const T*)a.A;
    const T* B = (const T*)a.B;

    TileLoader<T, AK, BM, BK, NT> la;
    TileLoader<T, BKC, BN, BK, NT> lb;

    typename MT::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < MT::NACC; ++e) acc[i][j][e] = 0.f;

    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (nk > 0) {
        la.load(A, a.lda, m0, a.M, kbeg, kend, tid);
        lb.load(B, a.ldb, n0, a.N, kbeg, kend, tid);
        la.template store<PITCH>(lds[0], tid);
        lb.template store<PITCH>(lds[0] + SA, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            la.load(A, a.lda, m0, a.M, kbeg + (kt + 1) * BK, kend, tid);
            lb.load(B, a.ldb, n0, a.N, kbeg + (kt + 1) * BK, kend, tid);
        }
        const T* sA = lds[cur] + (wm * TM * MTILE + MT::frag_row(lane)) * PITCH + MT::frag_k(lane);
        const T* sB = lds[cur] + SA + (wn * TN * MTILE + MT::frag_row(lane)) * PITCH + MT::frag_k(lane);
#pragma unroll
        for (int ks = 0; ks < BK / KSLICE; ++ks) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = ld16(sA + i * MTILE * PITCH + ks * KSLICE);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = ld16(sB + j * MTILE * PITCH + ks * KSLICE);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = MT::step(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
            la.template store<PITCH>(lds[cur ^ 1], tid);
            lb.template store<PITCH>(lds[cur ^ 1] + SA, tid);
        }
        __syncthreads();
    }

    float* wsC = nullptr;
    if constexpr (EPI == EPI_F32) wsC = (float*)a.C + (int64_t)blockIdx.z * split_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < MT::NACC; ++r) {
                const int row = m0 + wm * TM * MTILE + i * MTILE + MT::out_row(lane, r);
                const int col = n0 + wn * TN * MTILE + j * MTILE + MT::out_col(lane);
                epilogue_store<T, EPI>(a, wsC, row, col, acc[i][j][r]);
            }
}

// ---------------------------------------------------------------------------- bf16 kernel (LDS DMA)
// Operands go from global memory straight into LDS with gfx950's buffer loads to
// LDS (16 bytes per lane, no registers in between).  The buffer resource covers
// exactly the valid rows of each matrix, so reads past the end return zero and
// the K loop has no bounds checks.  One such load writes 64 consecutive 16-byte
// LDS slots (lane order); a tile's layout is chosen by which global chunk each
// lane fetches.  Two or three LDS stages: the loads for the next tiles are in
// flight while tile k is multiplied; one barrier per tile.
//   k-contiguous operand: LDS row = one mn index, BK k (64, or 32 in the
//     half-depth instance); the 16-byte chunk c of row r sits at slot c ^ swz(r).
//     Fragment reads: ds_read_b128.
//   mn-contiguous operand: LDS row = one k, ROWS mn values; chunk c of row k sits
//     at slot c ^ hsw(k).  Fragment reads: two ds_read_b64_tr_b16, which hand lane
//     j of each 16-lane group element e of the 8-byte word addressed by lane
//     4e + j/4 of that group (element j % 4 of it), i.e. a 4 x 16 transpose: with
//     lane i addressing (k0 + i/4, n0 + 4 (i%4)), lane j receives k0..k0+3 at n0 + j.
// Requirements (checked by the host): leading dimensions are multiples of 8
// elements, and a k-contiguous operand's columns between K and the next multiple
// of 64 read as zero (true when K % 64 == 0, or when the row padding holds zeros).


constexpr int GBK = 64;  // k per tile of the default (and every MX) instance

// k-contiguous tiles of BK k per row (BK / 8 chunks of 16 bytes): chunk c of row r
// sits at slot c ^ swz(r).  BK = 64: any 8 consecutive rows read at one logical
// chunk (fragment reads) and the 8 chunks of one row fall on distinct 16-byte bank
// groups.  BK = 32 (four rows per 256 bytes): any 4 consecutive rows, and rows
// r, r + 4, r + 8, r + 12, sit on distinct slots.  (Chosen by measurement among five
// slot patterns: the c_fc forward at 8192 x 3072 x 768 took 57.1 us against 59.4 with
// ((r >> 1) ^ (r >> 3)) & 3, which the counters showed losing 46 % of its LDS-active
// cycles to bank conflicts.)
template <int BK> __device__ __forceinline__ int swz(int r) {
    static_assert(BK == 64 || BK == 32, "k per tile");
    if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
    else return (r ^ (r >> 2)) & 3;
}
template <int BK> __device__ __forceinline__ int lds_pos(int r, int chunk) {
    return r * BK + ((chunk ^ swz<BK>(r)) << 3);
}
// mn-contiguous tiles (at least 16 chunks per row): chunk c of row k sits at slot
// c ^ 2 (k % 4) ^ 8 ((c / 2) % 2).  The 4 consecutive k rows one 16-lane group reads
// (32 bytes each) land on 4 distinct 32-byte bank groups, and the neighbouring group
// (the next 32 bytes of the same rows) on the other 128-byte half of the banks.
__device__ __forceinline__ int hsw(int k) { return (k & 3) << 1; }
__device__ __forceinline__ int mn_slot(int k, int c) { return c ^ hsw(k) ^ (((c >> 1) & 1) << 3); }
__device__ __forceinline__ int mn_chunk(int k, int slot) {
    return slot ^ hsw(k) ^ ((((slot >> 1) ^ k) & 1) << 3);
}


// Per-lane global offsets of one operand tile (ROWS mn x BK k) in 1 KB wave loads.
template <bool KC, int ROWS, int NW, int BK = GBK>
struct DmaTile {
    static constexpr int NI = ROWS * BK * 2 / 1024;  // wave loads per tile
    static_assert(NI % NW == 0, "wave loads per tile must divide among the waves");
    static constexpr int PW = NI / NW;
    static constexpr int CPR = ROWS / 8;           // mn-contiguous: chunks per k row
    static_assert(KC || CPR >= 16, "mn-contiguous tiles need at least 16 chunks per row");
    static constexpr int KCH = BK / 8;             // k-contiguous: chunks per mn row
    static constexpr int RPI = KC ? 64 / KCH : 64 / CPR;  // rows per wave load
    uint32_t voff[PW];
    uint32_t kstep;  // bytes per k element
    __device__ __forceinline__ void init(int wave, int lane, int row0, int64_t ld) {
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const int q = wave + NW * j;
            if constexpr (KC) {
                const int r = q * RPI + (int)((unsigned)lane / KCH);
                const int c = (lane & (KCH - 1)) ^ swz<BK>(r);
                voff[j] = (uint32_t)(((int64_t)(row0 + r) * ld + c * 8) * 2);
            } else {
                const int kr = q * RPI + lane / CPR;
                const int c = mn_chunk(kr, lane % CPR);
                voff[j] = (uint32_t)(((int64_t)kr * ld + row0 + c * 8) * 2);
            }
        }
        kstep = KC ? 2u : (uint32_t)(ld * 2);
    }
};


// `wtile`: LDS byte address of this wave's first 1 KB slot of the tile (an SGPR);
// the wave's loads go to slots wave, wave + NW, ...
template <int PW, int NW>
__device__ __forceinline__ void dma_issue(const dsc_t& d, uint32_t wtile, const uint32_t* voff, uint32_t soff) {
#pragma unroll
    for (int j = 0; j < PW; ++j) dma16(d, wtile + (uint32_t)(NW * j) * 1024u, voff[j], soff);
}

// Byte offsets in a tile of the MFMA fragment at mn offset f0, k slice ks
// (lane l: mn f0 + l % 32, k 16 ks + 8 (l / 32) .. +7).
template <bool KC, int ROWS, int BK = GBK>
__device__ __forceinline__ void frag_offsets(int lane, int f0, int ks, int* o) {
    if constexpr (KC) {
        o[0] = lds_pos<BK>(f0 + (lane & 31), 2 * ks + (lane >> 5)) * 2;
        o[1] = 0;
    } else {
        const int g = lane >> 4, i = lane & 15;
        const int col = f0 + 16 * (g & 1) + 4 * (i & 3);
        const int k = 16 * ks + 8 * (g >> 1) + (i >> 2);
        o[0] = k * ROWS * 2 + (mn_slot(k, col >> 3) << 4) + ((col >> 2) & 1) * 8;
        o[1] = o[0] + 4 * ROWS * 2;  // k + 4 (the slot depends on k % 4 only)
    }
}
template <bool KC>
__device__ __forceinline__ u32x4 frag_read(const bf16* tile, const int* o) {
    if constexpr (KC) {
        return *(const u32x4*)((const char*)tile + o[0]);
    } else {
        return read_tr2(tile, o[0], o[1]);
    }
}

// Tile of a block.  The grid is one-dimensional, rounded up to a multiple of 8.
// Blocks are dispatched round-robin over gfx950's 8 XCDs (block i on XCD i % 8),
// each with its own L2, so XCD x is given the contiguous run x * n/8 .. of the tile
// sequence, and that sequence walks groups of GROUP_M tile rows column by column: the
// blocks an XCD runs together share A row-tiles and B column-tiles in its L2
// instead of every XCD fetching every operand tile.  Returns false for padding.
// GROUP_M (measured on the step's shapes): 4 for products with at most 32 column tiles
// - the short-K qkv, c_fc and c_fc-input-gradient products 5-12 % faster than with 8,
// and with the half-depth weight-gradient instance the long-K ones too (tied-embedding
// dX 585 -> 554 us, -0.09 ms/step over two boxes) - and 8 for the vocabulary-wide
// lm_head forward.
__device__ __forceinline__ bool tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    constexpr int XCDS = 8;
    const int GROUP_M = tiles_n <= 32 ? 4 : 8;
    const int nt = tiles_m * tiles_n, per = (nt + XCDS - 1) / XCDS;
    const int t = (bid % XCDS) * per + bid / XCDS;
    if (t >= nt) return false;
    const int group = t / (GROUP_M * tiles_n), first = group * GROUP_M;
    const int gm = min(GROUP_M, tiles_m - first), idx = t - group * GROUP_M * tiles_n;
    tm = first + idx % gm;
    tn = idx / gm;
    return true;
}

// MX = true: the operands are MX FP8 (E4M3 codes, one E8M0 scale per 32 k) instead of
// bf16.  The tiles hold the same bytes (a 64-element bf16 k-tile is a 128-code MX
// k-tile), so loads, swizzles and fragment offsets are shared: k below counts 2-byte
// units.  v_mfma_scale_f32_32x32x64_f8f6f4 takes from lane l (group g = l / 32) the
// 16 bytes at k 16 g and the 16 at k 32 + 16 g of its 64-code slice - the fragments of
// two consecutive bf16 slices - and the scale of k-block g of its row (A) or column
// (B), one byte of a 32-bit register picked by op_sel.  Each stage also holds the
// scale words of its rows (1 KB for A, 1 KB for B), loaded by waves 0 and 1.
// XTRA: the bias epilogue's options (GemmArgs rope / swiglu / swiglu_gu) are compiled in
// only for the products that use them.
// BK: k per tile, 64, or 32 for the half-depth instance whose 72 KB of LDS and at most
// 128 registers per lane let two blocks share a CU (one block's epilogue then runs
// beside the other's main loop).
template <bool AK, bool BKC, int EPI, int BM, int BN, int WM, int WN, int ST = 2, bool MX = false, bool XTRA = false,
          int BK = GBK>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(BK == 32 ? 4 : 2)))
void gemm_bf16_kernel(GemmArgs a, int k_per_split, int64_t split_stride, uint32_t a_bytes, uint32_t b_bytes) {
    constexpr int NW = WM * WN, NT = 64 * NW;
    using MT = MfmaTraits<bf16>;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    static_assert(!MX || (AK && BKC && BM <= 256 && BN <= 256 && NW >= 2),
                  "MX: forward layout, <= 256 rows per scale load");
    constexpr int SCALE_ELEMS = MX ? 1024 : 0;  // 2 KB of scale words per stage
    constexpr int SA = BM * BK, STAGE = (BM + BN) * BK + SCALE_ELEMS;
    constexpr int LDS_ELEMS = ST * STAGE;
    __shared__ __attribute__((aligned(16))) bf16 lds[LDS_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    if (!tile_of_block(blockIdx.x, (a.M + BM - 1) / BM, (a.N + BN - 1) / BN, tm, tn)) return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * k_per_split;
    const int kend = min(a.K, kbeg + k_per_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const dsc_t ra = make_dsc(a.A, a_bytes), rb = make_dsc(a.B, b_bytes);
    // MX scale words: wave 0 loads A's, wave 1 B's (64 lanes x 16 bytes = 256 rows)
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // the wave index, known to be uniform
    dsc_t rsc{};
    uint32_t srow0 = 0, sstride = 0;
    if constexpr (MX) {
        const uint32_t nwords = (uint32_t)(a.K / GBK);  // scale words per row: one per 128 codes
        if (wv == 0) rsc = make_dsc(a.sa, nwords * (uint32_t)a.srows_a * 4u), srow0 = m0, sstride = (uint32_t)a.srows_a;
        if (wv == 1) rsc = make_dsc(a.sb, nwords * (uint32_t)a.srows_b * 4u), srow0 = n0, sstride = (uint32_t)a.srows_b;
    }
    // `wstage`: this wave's 1 KB slot address in the stage (stage base + wave KB), so
    // wave 0 lands on the A scale words and wave 1 on B's.  With 64-code k-tiles (BK =
    // 32) two consecutive tiles share a word; each stage holds its own copy.
    auto scale_issue = [&](uint32_t wstage, int ktile) {
        if constexpr (MX) {
            if (wv < 2)
                dma16(rsc, wstage + (uint32_t)((BM + BN) * BK * 2), (uint32_t)lane * 16u,
                      ((uint32_t)ktile / (GBK / BK) * sstride + srow0) * 4u);
        }
    };
    using TA = DmaTile<AK, BM, NW, BK>;
    using TB = DmaTile<BKC, BN, NW, BK>;
    TA ta;
    TB tb;
    ta.init(wave, lane, m0, a.lda);
    tb.init(wave, lane, n0, a.ldb);

    MT::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    int fa[TM][BK / 16][2], fb[TN][BK / 16][2];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i) frag_offsets<AK, BM, BK>(lane, (wm * TM + i) * 32, ks, fa[i][ks]);
#pragma unroll
        for (int j = 0; j < TN; ++j) frag_offsets<BKC, BN, BK>(lane, (wn * TN + j) * 32, ks, fb[j][ks]);
    }
    // Fragments of k-slice ks + 1 are read while the MFMAs of slice ks run.
    // `dma(ks)` issues the share of the next tile's loads that goes with k-slice ks.
    // MX: two 64-code MFMAs per stage, each on the fragments of bf16 slices 2 s and
    // 2 s + 1; lane group g's scale byte for k-block 2 s + g of the stage is byte 2 s
    // of its row's stage word shifted right by 8 g.
    auto compute_mx = [&](const bf16* st, auto&& dma) {
        typedef int v8i __attribute__((ext_vector_type(8)));
        const uint32_t* swa = (const uint32_t*)(st + (BM + BN) * BK);
        const uint32_t* swb = swa + 256;
        const int sh = 8 * (lane >> 5);
        uint32_t sca[TM], scb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) sca[i] = swa[(wm * TM + i) * 32 + (lane & 31)] >> sh;
#pragma unroll
        for (int j = 0; j < TN; ++j) scb[j] = swb[(wn * TN + j) * 32 + (lane & 31)] >> sh;
        v8i xa[2][TM], xb[2][TN];
        auto rd = [&](int buf, int sl) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const u32x4 lo = frag_read<AK>(st, fa[i][2 * sl]), hi = frag_read<AK>(st, fa[i][2 * sl + 1]);
                xa[buf][i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const u32x4 lo = frag_read<BKC>(st + SA, fb[j][2 * sl]), hi = frag_read<BKC>(st + SA, fb[j][2 * sl + 1]);
                xb[buf][j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        };
        rd(0, 0);
        rd(1, 1);
        dma(0);
        dma(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[0][i], xb[0][j], acc[i][j], 0, 0, 0,
                                                                            (int)sca[i], 0, (int)scb[j]);
        dma(2);
        dma(3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[1][i], xb[1][j], acc[i][j], 0, 0, 2,
                                                                            (int)sca[i], 2, (int)scb[j]);
    };
    // MX with 64-code k-tiles: one MFMA k-slice per stage, on half `par` of the rows'
    // 128-code scale words (lane group g's byte 2 par + g, brought to byte 0).
    auto compute_mx64 = [&](const bf16* st, int par, auto&& dma) {
        typedef int v8i __attribute__((ext_vector_type(8)));
        const uint32_t* swa = (const uint32_t*)(st + (BM + BN) * BK);
        const uint32_t* swb = swa + 256;
        const int sh = 8 * (lane >> 5) + 16 * par;
        uint32_t sca[TM], scb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) sca[i] = swa[(wm * TM + i) * 32 + (lane & 31)] >> sh;
#pragma unroll
        for (int j = 0; j < TN; ++j) scb[j] = swb[(wn * TN + j) * 32 + (lane & 31)] >> sh;
        v8i xa[TM], xb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const u32x4 lo = frag_read<AK>(st, fa[i][0]), hi = frag_read<AK>(st, fa[i][1]);
            xa[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const u32x4 lo = frag_read<BKC>(st + SA, fb[j][0]), hi = frag_read<BKC>(st + SA, fb[j][1]);
            xb[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
        dma(0);
        dma(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[i], xb[j], acc[i][j], 0, 0, 0,
                                                                            (int)sca[i], 0, (int)scb[j]);
    };
    auto compute = [&](const bf16* st, auto&& dma) {
        u32x4 xa[2][TM], xb[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) xa[0][i] = frag_read<AK>(st, fa[i][0]);
#pragma unroll
        for (int j = 0; j < TN; ++j) xb[0][j] = frag_read<BKC>(st + SA, fb[j][0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cb = ks & 1, nb = cb ^ 1;
            if (ks + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < TM; ++i) xa[nb][i] = frag_read<AK>(st, fa[i][ks + 1]);
#pragma unroll
                for (int j = 0; j < TN; ++j) xb[nb][j] = frag_read<BKC>(st + SA, fb[j][ks + 1]);
            }
            dma(ks);
            __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this slice's MFMAs
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = MT::step(xa[cb][i], xb[cb][j], acc[i][j]);
        }
    };

    // ST-stage ring: tiles kt+1 .. kt+ST-1 are in flight while tile kt is multiplied
    constexpr int LPT = TA::PW + TB::PW;  // wave loads per tile
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds) + (uint32_t)wave * 1024u);  // this wave
#pragma unroll
    for (int s0 = 0; s0 < ST - 1; ++s0)
        if (s0 < nk) {
            const uint32_t k1 = (uint32_t)(kbeg + s0 * BK);
            scale_issue(lbase + s0 * STAGE * 2, kbeg / BK + s0);
            dma_issue<TA::PW, NW>(ra, lbase + s0 * STAGE * 2, ta.voff, k1 * ta.kstep);
            dma_issue<TB::PW, NW>(rb, lbase + (s0 * STAGE + SA) * 2, tb.voff, k1 * tb.kstep);
        }
    // Row sums of op(A) (the bias gradient of a weight-gradient product), taken by
    // the blocks of the first column tile from the A tiles in LDS: thread t owns the
    // 8 m values of chunk t % RCPR and adds the k rows t / RCPR + RROWS p.
    constexpr bool RS = !AK && EPI == EPI_F32;
    constexpr int RCPR = BM / 8, RROWS = NT / RCPR;
    static_assert(!RS || (NT % RCPR == 0 && BK % RROWS == 0), "row-sum thread mapping");
    const bool do_rs = RS && a.rowsum && n0 == 0;
    float rs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rs[e] = 0.f;

    int cur = 0;  // stage of tile kt
    for (int kt = 0; kt < nk; ++kt) {
        // tile kt has landed (every wave waits for its own loads, then the barrier);
        // every wave is also done with tile kt-1, whose stage the next loads reuse
        if (kt + ST - 2 < nk) wait_loads<LPT * (ST - 2)>();
        else wait_loads<0>();
        __builtin_amdgcn_s_barrier();
        // The next tile's loads: with three or more stages they go out spread over this
        // tile's k-slices (evening out the load and LDS-write traffic); with two, the
        // one tile of slack is needed and they all go out first.
        constexpr int SPREAD = ST >= 3 ? BK / 16 : 1;
        const bool more = kt + ST - 1 < nk;
        const int nst = cur == 0 ? ST - 1 : cur - 1;
        const uint32_t nxt = lbase + (uint32_t)(nst * STAGE * 2);
        const uint32_t k1 = (uint32_t)(kbeg + (kt + ST - 1) * BK);
        auto dma = [&](int ks) {
            if (!more) return;
            if (ks == 0) scale_issue(nxt, kbeg / BK + kt + ST - 1);
#pragma unroll
            for (int j = 0; j < TA::PW; ++j)
                if (j % SPREAD == ks) dma16(ra, nxt + (uint32_t)(NW * j) * 1024u, ta.voff[j], k1 * ta.kstep);
#pragma unroll
            for (int j = 0; j < TB::PW; ++j)
                if ((TA::PW + j) % SPREAD == ks)
                    dma16(rb, nxt + (uint32_t)(SA * 2 + NW * j * 1024), tb.voff[j], k1 * tb.kstep);
        };
        if constexpr (RS) {
            if (do_rs) {
                const bf16* at = lds + cur * STAGE;
                const int c = tid % RCPR;
#pragma unroll
                for (int p = 0; p < BK / RROWS; ++p) {
                    const int kr = tid / RCPR + p * RROWS;
                    float v[8];
                    unpack16<bf16>(*(const u32x4*)(at + kr * BM + mn_slot(kr, c) * 8), v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) rs[e] += v[e];
                }
            }
        }
        if constexpr (MX && BK == 32) compute_mx64(lds + cur * STAGE, (kbeg / BK + kt) & 1, dma);
        else if constexpr (MX) compute_mx(lds + cur * STAGE, dma);
        else compute(lds + cur * STAGE, dma);
        cur = cur + 1 == ST ? 0 : cur + 1;
    }
    __syncthreads();
    if constexpr (RS) {
        if (do_rs) {  // block-uniform
            float* red = (float*)lds;
            const int c = tid % RCPR, g = tid / RCPR;
#pragma unroll
            for (int e = 0; e < 8; ++e) red[g * BM + c * 8 + e] = rs[e];
            __syncthreads();
            if (tid < BM && m0 + tid < a.M) {
                float v = 0.f;
                for (int h = 0; h < RROWS; ++h) v += red[h * BM + tid];
                a.rowsum[blockIdx.z * split_stride + m0 + tid] = v;
            }
            __syncthreads();
        }
    }

    // Epilogue through LDS: the accumulators are written as fp32 rows [row][BN + 8]
    // (the pad puts the two half-waves of a 32x32 tile on different banks), then
    // each thread takes 8 consecutive columns of a row, applies the fused epilogue
    // and writes 16-byte vectors.  A thread keeps the same 8 columns for the whole
    // tile, so its bias values are loaded once; the residual / GELU-input rows of a
    // pass are all requested before the first is used.  Tiles taller than the LDS
    // allows go in passes.
    constexpr int EP = BN + 8;
    constexpr int LDS_BYTES = LDS_ELEMS * 2;
    constexpr int NPASS = (BM * EP * 4 <= LDS_BYTES) ? 1 : (BM / 2 * EP * 4 <= LDS_BYTES) ? 2 : 4;
    constexpr int EROWS = BM / NPASS;
    static_assert(EROWS * NPASS == BM && EROWS % 32 == 0, "epilogue pass split");
    constexpr int CPR = BN / 8;  // 8-column chunks per row
    static_assert(NT % CPR == 0 && (EROWS * CPR) % NT == 0, "epilogue chunk mapping");
    constexpr int ITER = EROWS * CPR / NT, RSTEP = NT / CPR;
    constexpr bool NEED_R = EPI == EPI_BIAS_RES || EPI == EPI_GELU_BWD;
    const int lc = (tid % CPR) * 8, lr0 = tid / CPR;
    const int col = n0 + lc;
    const bool colok = col < a.N, full = col + 8 <= a.N;
    float bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[e] = 0.f;
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_RES || EPI == EPI_BIAS_GELU) {
        if (a.bias && colok) {
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = (col + e < a.N) ? a.bias[col + e] : 0.f;
        }
    }
    float* ebuf = (float*)lds;
    float* wsC = nullptr;
    if constexpr (EPI == EPI_F32) wsC = (float*)a.C + (int64_t)blockIdx.z * split_stride;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int r0 = pass * EROWS;
        u32x4 rr[NEED_R ? ITER : 1];
        if constexpr (NEED_R) {
#pragma unroll
            for (int it = 0; it < ITER; ++it) {
                const int row = m0 + r0 + lr0 + it * RSTEP;
                rr[it] = (row < a.M && full) ? ld16((const bf16*)a.R + (int64_t)row * a.ldc + col) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int trow = (wm * TM + i) * 32;  // tile-local first row of this MFMA block
            if (trow >= r0 && trow < r0 + EROWS) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ebuf[(trow - r0 + MT::out_row(lane, r)) * EP + (wn * TN + j) * 32 + MT::out_col(lane)] =
                            acc[i][j][r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int lr = lr0 + it * RSTEP;
            const int row = m0 + r0 + lr;
            if (row >= a.M || !colok) continue;
            float v[8];
            const float4 v0 = *(const float4*)(ebuf + lr * EP + lc);
            const float4 v1 = *(const float4*)(ebuf + lr * EP + lc + 4);
            v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
            v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
            const int64_t o = (int64_t)row * a.ldc + col;
            if constexpr (EPI == EPI_F32) {
                if (full) {
                    *(float4*)(wsC + o) = v0;
                    *(float4*)(wsC + o + 4) = v1;
                } else {
                    for (int e = 0; e < 8 && col + e < a.N; ++e) wsC[o + e] = v[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += bv[e];
                if constexpr (EPI == EPI_BIAS && XTRA) {
                    if (a.rope && full && col < a.rope_cols) {  // col and rope_hs are multiples of 8
                        const float2* tr =
                            a.rope + (int64_t)(row % a.rope_period) * (a.rope_hs / 2) + (col % a.rope_hs) / 2;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float2 cs = tr[j];
                            const float x0 = v[2 * j], x1 = v[2 * j + 1];
                            v[2 * j] = x0 * cs.x - x1 * cs.y;
                            v[2 * j + 1] = x0 * cs.y + x1 * cs.x;
                        }
                    }
                }
                float rv[8];
                if constexpr (NEED_R) {
                    if (full) unpack16<bf16>(rr[it], rv);
                    else
                        for (int e = 0; e < 8; ++e) rv[e] = (col + e < a.N) ? to_f32(((const bf16*)a.R)[o + e]) : 0.f;
                }
                float out2[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (EPI == EPI_BIAS_RES) v[e] += rv[e];
                    if constexpr (EPI == EPI_BIAS_GELU) out2[e] = gelu_fwd(v[e]);
                    if constexpr (EPI == EPI_GELU_BWD) v[e] *= gelu_bwd(rv[e]);
                }
                bf16* C = (bf16*)a.C;
                if constexpr (EPI == EPI_BIAS && XTRA) {
                    if (a.swiglu_gu && full) {  // SwiGLU backward: 8 hidden units' dh -> 16 (dg, du)
                        const int64_t o2 = (int64_t)row * 2 * a.ld_swiglu + 2 * col;
                        float gu[16], d[16];
                        unpack16<bf16>(ld16(a.swiglu_gu + o2), gu);
                        unpack16<bf16>(ld16(a.swiglu_gu + o2 + 8), gu + 8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float g = gu[2 * e], u = gu[2 * e + 1], sg = 1.f / (1.f + __expf(-g));
                            d[2 * e] = v[e] * u * sg * (1.f + g * (1.f - sg));
                            d[2 * e + 1] = v[e] * g * sg;
                        }
                        st16(a.swiglu + o2, pack16<bf16>(d));
                        st16(a.swiglu + o2 + 8, pack16<bf16>(d + 8));
                        continue;
                    }
                }
                if (full) {
                    // the vocabulary-sized logits (the only 256-row tiles with a plain bias):
                    // non-temporal stores, so the 0.8 GB they take does not displace the
                    // operands from the caches (702 -> 636 us, and the softmax-CE that reads
                    // them 332 -> 313 us)
                    if constexpr (BM == 256 && EPI == EPI_BIAS) __builtin_nontemporal_store(pack16<bf16>(v), (u32x4*)(C + o));
                    // the GELU input, read again only by the backward pass: non-temporal too,
                    // so the GELU output stays cached for the product that reads it next
                    // (c_fc projection forward 52.7 -> 50.6 us in the step, -0.04 ms/step)
                    else if constexpr (EPI == EPI_BIAS_GELU) __builtin_nontemporal_store(pack16<bf16>(v), (u32x4*)(C + o));
                    else st16(C + o, pack16<bf16>(v));
                    if constexpr (EPI == EPI_GELU_BWD) {
                        // MX codes of the stored output (the next input-gradient product's
                        // upstream gradient), grouped as for the GELU output below
                        if (a.q2) {
                            float t[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) t[e] = v[e];
                            round_bf16_8(t);
                            uint32_t cw[2];
                            const uint32_t word = mx_stage_word(mx_quant8(t, cw));
                            *(uint2*)(a.q2 + (int64_t)row * a.ldq2 + col) = make_uint2(cw[0], cw[1]);
                            if ((tid & 15) == 0) *(uint32_t*)(a.s2 + ((int64_t)(col / 128) * a.M + row) * 4) = word;
                        }
                    }
                    if constexpr (EPI == EPI_BIAS && XTRA) {
                        if (a.swiglu) {  // 4 (gate, up) pairs -> 4 hidden units
                            float gu[8], h[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) gu[e] = v[e];
                            round_bf16_8(gu);
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const float g = gu[2 * j];
                                h[j] = g / (1.f + __expf(-g)) * gu[2 * j + 1];
                                h[4 + j] = 0.f;
                            }
                            const u32x4 pk = pack16<bf16>(h);
                            *(uint2*)(a.swiglu + (int64_t)row * a.ld_swiglu + col / 2) = make_uint2(pk[0], pk[1]);
                        }
                    }
                    if constexpr (EPI == EPI_BIAS_GELU) {
                        st16((bf16*)a.C2 + o, pack16<bf16>(out2));
                        // MX codes of the stored GELU output: 4 consecutive threads hold a
                        // 32-block, 16 a 128-column stage (the host asks for this only when
                        // N % 128 == 0, so a 16-thread group is wholly inside or outside N)
                        if (a.q2) {
                            round_bf16_8(out2);
                            uint32_t cw[2];
                            const uint32_t word = mx_stage_word(mx_quant8(out2, cw));
                            *(uint2*)(a.q2 + (int64_t)row * a.ldq2 + col) = make_uint2(cw[0], cw[1]);
                            if ((tid & 15) == 0) *(uint32_t*)(a.s2 + ((int64_t)(col / 128) * a.M + row) * 4) = word;
                        }
                    }
                } else {
                    for (int e = 0; e < 8 && col + e < a.N; ++e) {
                        C[o + e] = from_f32<bf16>(v[e]);
                        if constexpr (EPI == EPI_BIAS_GELU) ((bf16*)a.C2)[o + e] = from_f32<bf16>(out2[e]);
                    }
                }
            }
        }
        if (pass + 1 < NPASS) __syncthreads();
    }
}

// Profiler name of a launch: layout, epilogue and shape (M x N x K, / splits),
// interned so the pointer stays valid.
template <class T, bool AK, bool BKC, int EPI>
static const char* gemm_name(int M, int N, int K, int splits) {
    static std::mutex mu;
    static std::set<std::string> names;
    std::string n = std::string("gemm_") + (sizeof(T) == 2 ? "bf16_" : "f32_") +
                    (AK && BKC ? "xwT" : AK ? "dyW" : "dyTx") + "_" +
                    (EPI == EPI_BIAS ? "bias" : EPI == EPI_BIAS_RES ? "bias_res" :
                     EPI == EPI_BIAS_GELU ? "bias_gelu" : EPI == EPI_GELU_BWD ? "gelu_bwd" : "f32out") +
                    "_" + std::to_string(M) + "x" + std::to_string(N) + "x" + std::to_string(K);
    if (splits > 1) n += "/" + std::to_string(splits);
    std::lock_guard<std::mutex> lk(mu);
    return names.insert(n).first->c_str();
}

static bool use_tile256(int M, int N, int splits) {
    return (int64_t)((M + 255) / 256) * ((N + 255) / 256) * splits >= 768;
}


template <class T, bool AK, bool BKC, int EPI>
static hipError_t launch(const GemmArgs& a, int splits, int k_per_split, int64_t split_stride, hipStream_t s) {
    const double es = sizeof(T), mn = (double)a.M * a.N;
    const double out_bytes = EPI == EPI_F32 ? 4 * mn : (EPI == EPI_BIAS ? es * mn : 2 * es * mn);
    ProfScope prof(s, gemm_name<T, AK, BKC, EPI>(a.M, a.N, a.K, splits), 2.0 * mn * a.K,
                   es * ((double)a.M + a.N) * a.K + out_bytes);
    if constexpr (sizeof(T) == 2) {
        // buffer extents in bytes: whole rows of each operand as stored
        const int64_t ab = (AK ? (int64_t)a.M : (int64_t)a.K) * a.lda * 2;
        const int64_t bb = (BKC ? (int64_t)a.N : (int64_t)a.K) * a.ldb * 2;
        if (ab >= (int64_t)1 << 32 || bb >= (int64_t)1 << 32) return hipErrorInvalidValue;
        // Tile shapes (both 8 waves, measured on the step's shapes): 256 x 256 with
        // waves of 128 x 64 and two stages when there are at least three such tiles
        // per CU; otherwise 128 x 256 with waves of 64 x 64 and three stages.  Both
        // hold one block per CU (128 / 144 KB of LDS).
        if constexpr (EPI == EPI_BIAS) {
            if (a.rope || a.swiglu) {  // the extras' instance (128 x 256 tiles)
                const int nt = ((a.N + 255) / 256) * ((a.M + 127) / 128);
                dim3 grid((nt + 7) / 8 * 8, 1, splits);
                hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, EPI, 128, 256, 2, 4, 3, false, true>), grid, dim3(512), 0,
                                   s, a, k_per_split, split_stride, (uint32_t)ab, (uint32_t)bb);
                return hipGetLastError();
            }
        }
        // GELU epilogues (c_fc forward, the GELU-input gradient) with at least 384
        // 128 x 256 tiles: the half-depth instance (72 KB of LDS, 4 waves per SIMD)
        // runs two blocks per CU, so one block's epilogue overlaps the other's main
        // loop (GELU-input gradient at 8192 x 3072 x 768: 59.6 -> 50.4 us, same bits;
        // 384 takes in the forward pass's half-batch c_fc products, which run two at a
        // time).  Products with fewer tiles or a long K are slower with it (up to 24 %).
        if constexpr (AK && (EPI == EPI_GELU_BWD || EPI == EPI_BIAS_GELU)) {
            const int nt = ((a.N + 255) / 256) * ((a.M + 127) / 128);
            if (splits == 1 && nt >= 384) {
                hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, EPI, 128, 256, 2, 4, 3, false, false, 32>),
                                   dim3((nt + 7) / 8 * 8), dim3(512), 0, s, a, k_per_split, split_stride,
                                   (uint32_t)ab, (uint32_t)bb);
                return hipGetLastError();
            }
        }
        // Weight gradients (the second stream's products, fp32 out) use the half-depth
        // instance as well: its 72 KB of LDS leave room on the CU for the first
        // stream's attention and LayerNorm blocks (-0.05 ms/step; alone they are up to
        // 13 % slower, with their blocks packed two to a CU).
        if constexpr (!AK && EPI == EPI_F32) {
            const int nt = ((a.N + 255) / 256) * ((a.M + 127) / 128);
            hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, EPI, 128, 256, 2, 4, 3, false, false, 32>),
                               dim3((nt + 7) / 8 * 8, 1, splits), dim3(512), 0, s, a, k_per_split, split_stride,
                               (uint32_t)ab, (uint32_t)bb);
            return hipGetLastError();
        }
        if (splits == 1 && use_tile256(a.M, a.N, 1)) {
            const int nt = ((a.N + 255) / 256) * ((a.M + 255) / 256);
            dim3 grid((nt + 7) / 8 * 8, 1, splits);
            hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, EPI, 256, 256, 2, 4, 2>), grid, dim3(512), 0, s, a,
                               k_per_split, split_stride, (uint32_t)ab, (uint32_t)bb);
        } else {
            const int nt = ((a.N + 255) / 256) * ((a.M + 127) / 128);
            dim3 grid((nt + 7) / 8 * 8, 1, splits);
            hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, EPI, 128, 256, 2, 4, 3>), grid, dim3(512), 0, s, a,
                               k_per_split, split_stride, (uint32_t)ab, (uint32_t)bb);
        }
    } else {
        constexpr int BM = 128, BN = 128, BK = 32, WM = 2, WN = 2;
        dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, splits);
        hipLaunchKernelGGL((gemm_kernel<T, AK, BKC, EPI, BM, BN, BK, WM, WN>), grid, dim3(64 * WM * WN), 0, s, a,
                           k_per_split, split_stride);
    }
    return hipGetLastError();
}

template <class T, int EPI>
static hipError_t dispatch_layout(const GemmArgs& a, bool ak, bool bk, int splits, int kps, int64_t ss,
                                  hipStream_t s) {
    if (ak && bk) return launch<T, true, true, EPI>(a, splits, kps, ss, s);
    if (ak && !bk) return launch<T, true, false, EPI>(a, splits, kps, ss, s);
    if (!ak && !bk) return launch<T, false, false, EPI>(a, splits, kps, ss, s);
    return hipErrorInvalidValue;  // (m-contiguous A, k-contiguous B) is not used by the step
}

template <class T>
hipError_t gemm(const GemmArgs& a, bool ak, bool bk, int epi, float* ws, size_t ws_floats, hipStream_t s) {
    constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    const bool extras = a.rope || a.swiglu;
    // the forward extras need the (x, W^T) layout; the SwiGLU backward rides on dh = dY W
    if (extras && (sizeof(T) != 2 || epi != EPI_BIAS || !ak || (bk && a.swiglu_gu) || (!bk && !a.swiglu_gu) ||
                   a.N % 8))
        return hipErrorInvalidValue;
    if constexpr (sizeof(T) == 2) {
        // 16-byte rows, and k-contiguous operands readable (zero-padded) up to a multiple of 64
        if (a.lda % 8 || a.ldb % 8 || a.ldc % 8) return hipErrorInvalidValue;
        const int64_t kpad = (a.K + 63) / 64 * 64;
        if ((ak && a.lda < kpad) || (bk && a.ldb < kpad)) return hipErrorInvalidValue;
    }
    if (epi == EPI_F32) {
        // Output fp32 [M, N] with row stride ldc.  Few output tiles and a long K:
        // split K over blockIdx.z into fp32 partials in `ws`, then reduce in a fixed
        // order.  bf16: one 128 x 256 block per CU, so aim at 256 blocks; fp32: 128 x
        // 128 tiles, two per CU.  Each split keeps at least 8 k-tiles.
        const int tiles = sizeof(T) == 2 ? ((a.M + 127) / 128) * ((a.N + 255) / 256)
                                         : ((a.M + 127) / 128) * ((a.N + 127) / 128);
        const int slots = sizeof(T) == 2 ? 256 : 512;
        // With row sums, each split's partials are [M x N | M], so the sums of the
        // bias gradient stored right after its weight gradient reduce in the same pass.
        if (a.rowsum && (sizeof(T) != 2 || ak)) return hipErrorInvalidValue;
        const int64_t mn = (int64_t)a.M * a.N, ss = mn + (a.rowsum ? (a.M + 3) / 4 * 4 : 0);
        int splits = 1;
        if (ws && a.ldc == a.N && tiles < slots && !(sizeof(T) == 2 && use_tile256(a.M, a.N, 1))) {
            splits = slots / tiles;
            splits = std::min(splits, a.K / (8 * BK));
            while (splits > 1 && (size_t)splits * ss > ws_floats) --splits;
            splits = std::max(splits, 1);
        }
        if (splits == 1) return dispatch_layout<T, EPI_F32>(a, ak, bk, 1, a.K, 0, s);
        int kps = (a.K + splits - 1) / splits;
        kps = (kps + BK - 1) / BK * BK;
        splits = (a.K + kps - 1) / kps;
        GemmArgs p = a;
        p.C = ws;
        if (a.rowsum) p.rowsum = ws + mn;
        hipError_t e = dispatch_layout<T, EPI_F32>(p, ak, bk, splits, kps, ss, s);
        if (e != hipSuccess) return e;
        if (a.rowsum && a.rowsum == (float*)a.C + mn)
            return splitk_reduce((float*)a.C, ws, splits, mn + a.M, ss, s);
        e = splitk_reduce((float*)a.C, ws, splits, mn, ss, s);
        if (e != hipSuccess || !a.rowsum) return e;
        return splitk_reduce(a.rowsum, ws + mn, splits, a.M, ss, s);
    }
    if constexpr (sizeof(T) == 2) {
        // bf16 output with too few 128 x 256 tiles to fill the chip and a long K (the
        // tied-embedding dX): split K so the blocks fill whole waves of 256, then sum
        // the fp32 partials and add the bias in a fixed order.
        const int tiles = ((a.M + 127) / 128) * ((a.N + 255) / 256);
        if (epi == EPI_BIAS && ws && !extras && tiles < 256 && a.K >= 4096 && a.N % 8 == 0) {
            auto eff = [&](int sp) { return (double)tiles * sp / (((tiles * sp + 255) / 256) * 256.0); };
            int best = 1;
            for (int sp = 2; sp <= 8; ++sp)
                if (eff(sp) > eff(best) + 0.1 && (size_t)sp * a.M * a.N <= ws_floats) best = sp;
            if (best > 1) {
                int kps = (a.K + best - 1) / best;
                kps = (kps + BK - 1) / BK * BK;
                const int splits = (a.K + kps - 1) / kps;
                GemmArgs p = a;
                p.C = ws;
                p.ldc = a.N;
                p.bias = nullptr;
                p.rowsum = nullptr;
                hipError_t e = dispatch_layout<T, EPI_F32>(p, ak, bk, splits, kps, (int64_t)a.M * a.N, s);
                if (e != hipSuccess) return e;
                return splitk_reduce_bf16((bf16*)a.C, a.ldc, ws, splits, a.M, a.N, a.bias, s);
            }
        }
    }
    switch (epi) {
        case EPI_BIAS: return dispatch_layout<T, EPI_BIAS>(a, ak, bk, 1, a.K, 0, s);
        case EPI_BIAS_RES: return dispatch_layout<T, EPI_BIAS_RES>(a, ak, bk, 1, a.K, 0, s);
        case EPI_BIAS_GELU: return dispatch_layout<T, EPI_BIAS_GELU>(a, ak, bk, 1, a.K, 0, s);
        case EPI_GELU_BWD: return dispatch_layout<T, EPI_GELU_BWD>(a, ak, bk, 1, a.K, 0, s);
    }
    return hipErrorInvalidValue;
}

template <int EPI>
static hipError_t launch_mx(const GemmArgs& e, int K, uint32_t ab, uint32_t bb, hipStream_t s) {
    static std::mutex mu;
    static std::set<std::string> names;
    const char* name;
    {
        std::string n = std::string("gemm_mxfp8_xwT_") +
                        (EPI == EPI_BIAS ? "bias" : EPI == EPI_BIAS_RES ? "bias_res" :
                         EPI == EPI_BIAS_GELU ? "bias_gelu" : "gelu_bwd") + "_" +
                        std::to_string(e.M) + "x" + std::to_string(e.N) + "x" + std::to_string(K);
        std::lock_guard<std::mutex> lk(mu);
        name = names.insert(n).first->c_str();
    }
    const double mn = (double)e.M * e.N;
    const double out_bytes = EPI == EPI_BIAS ? 2 * mn : 4 * mn;
    ProfScope prof(s, name, 2.0 * mn * K, ((double)e.M + e.N) * K * (1.0 + 1.0 / 32) + out_bytes);
    // The bf16 128 x 256 tile with three stages (150 KB of LDS with the scale words).
    // The 256 x 256 tile does not fit: an MX operand fragment is twice a bf16 one, and
    // its 128 x 64 wave tiles would spill.
    const int nt = ((e.N + 255) / 256) * ((e.M + 127) / 128);
    if constexpr (EPI == EPI_BIAS) {
        if (e.rope || e.swiglu) {
            hipLaunchKernelGGL((gemm_bf16_kernel<true, true, EPI, 128, 256, 2, 4, 3, true, true>),
                               dim3((nt + 7) / 8 * 8), dim3(512), 0, s, e, e.K, (int64_t)0, ab, bb);
            return hipGetLastError();
        }
    }
    // The GELU epilogues with at least 384 tiles: 64-code k-tiles (78 KB of LDS, at
    // most 128 registers), two blocks per CU, as for the bf16 products.
    if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_GELU_BWD) {
        if (nt >= 384) {
            hipLaunchKernelGGL((gemm_bf16_kernel<true, true, EPI, 128, 256, 2, 4, 3, true, false, 32>),
                               dim3((nt + 7) / 8 * 8), dim3(512), 0, s, e, e.K, (int64_t)0, ab, bb);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, EPI, 128, 256, 2, 4, 3, true>), dim3((nt + 7) / 8 * 8),
                       dim3(512), 0, s, e, e.K, (int64_t)0, ab, bb);
    return hipGetLastError();
}

hipError_t gemm_mx(const GemmArgs& a, int epi, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.q2 && ((epi != EPI_BIAS_GELU && epi != EPI_GELU_BWD) || a.N % 128 || !a.s2 || a.ldq2 < a.N || a.ldq2 % 16))
        return hipErrorInvalidValue;
    if (a.K <= 0 || a.K % 128 || a.lda % 16 || a.ldb % 16 || a.ldc % 8 || a.lda < a.K || a.ldb < a.K)
        return hipErrorInvalidValue;
    if (!a.A || !a.B || !a.C || !a.sa || !a.sb || a.srows_a < a.M || a.srows_b < a.N) return hipErrorInvalidValue;
    if ((epi == EPI_BIAS_RES || epi == EPI_GELU_BWD) && !a.R) return hipErrorInvalidValue;
    if (epi == EPI_BIAS_GELU && !a.C2) return hipErrorInvalidValue;
    if (epi == EPI_GELU_BWD && a.bias) return hipErrorInvalidValue;
    const int64_t ab = (int64_t)a.M * a.lda, bb = (int64_t)a.N * a.ldb;
    const int64_t sab = (int64_t)(a.K / 128) * a.srows_a * 4, sbb = (int64_t)(a.K / 128) * a.srows_b * 4;
    if (ab >= (int64_t)1 << 32 || bb >= (int64_t)1 << 32 || sab >= (int64_t)1 << 32 || sbb >= (int64_t)1 << 32)
        return hipErrorInvalidValue;
    // the kernel counts k and leading dimensions in 2-byte units (two codes)
    GemmArgs e = a;
    e.K = a.K / 2;
    e.lda = a.lda / 2;
    e.ldb = a.ldb / 2;
    e.rowsum = nullptr;
    switch (epi) {
        case EPI_BIAS: return launch_mx<EPI_BIAS>(e, a.K, (uint32_t)ab, (uint32_t)bb, s);
        case EPI_BIAS_RES: return launch_mx<EPI_BIAS_RES>(e, a.K, (uint32_t)ab, (uint32_t)bb, s);
        case EPI_BIAS_GELU: return launch_mx<EPI_BIAS_GELU>(e, a.K, (uint32_t)ab, (uint32_t)bb, s);
        case EPI_GELU_BWD: return launch_mx<EPI_GELU_BWD>(e, a.K, (uint32_t)ab, (uint32_t)bb, s);
    }
    return hipErrorInvalidValue;
}

template hipError_t gemm<float>(const GemmArgs&, bool, bool, int, float*, size_t, hipStream_t);
template hipError_t gemm<bf16>(const GemmArgs&, bool, bool, int, float*, size_t, hipStream_t);

}  // namespace gpt2
