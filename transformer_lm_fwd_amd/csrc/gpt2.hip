// Host side of the GPT-2 training-step library: arena layout and the C ABI
// entry points declared in include/gpt2.h.  Every step of the path runs in the
// kernels of this directory; this file only validates, lays out and enqueues.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

using namespace gpt2;

namespace {

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
    g_error = msg;
    return code;
}

}  // namespace

int gpt2::report_error(int code, const char* msg) { return fail(code, msg); }

namespace {

enum { P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_PROJW, P_PROJB, P_LN2W, P_LN2B, P_FCW, P_FCB, P_FCPW, P_FCPB, P_N };

struct LayerActs {
    size_t ln1, ln1s, qkv, atty, lse, res2, ln2, ln2s, fch, fchg, res3;
};

}  // namespace

struct gpt2_arena {
    gpt2_config cfg;
    int B, T, dtype, Vp, hs;
    // block type: GPT2_BLOCK_GPT2, or GPT2_BLOCK_LLAMA (RMSNorm, no biases, SwiGLU MLP of
    // width H, rotary positions); F1 / F2: widths of the MLP's first product / activation
    int block = GPT2_BLOCK_GPT2;
    int64_t H = 0, F1 = 0, F2 = 0;
    bool rope_ready = false;  // the rotary table has been built
    int64_t nparams;
    char* base;
    size_t bytes;
    size_t act_size;  // bytes per activation element
    // parameter element offsets
    int64_t o_wte, o_wpe, o_lnfw, o_lnfb;
    std::vector<int64_t> o_layer;  // [L * P_N]
    // byte offsets of regions
    size_t params, grads, adam_m, adam_v, params16;
    size_t encoded, lnf, lnfs, logits, losses, loss;
    std::vector<LayerActs> la;
    size_t dres[4], dbuf, dqkv[2], dfch[2], dh, dsum, partial, partial_side, ws, ws_main, census;
    size_t partial_floats, ws_floats, ws_main_floats;
    bool loss_ready;
    bool census_armed = false;  // the token census holds its idle state (set by the first backward)
    const int32_t* inputs;
    // Concurrency: parameter-gradient work of the backward pass and one half of a split
    // forward pass run on `side`.  rd_* mark the side stream's last read of each ring
    // buffer; fork events order side work after main-stream producers.  The stream is
    // the caller's (gpt2_set_side_stream) or, failing that, created on first use.
    hipStream_t side = nullptr;
    bool side_owned = false;
    bool events_ready = false;
    hipEvent_t rd_res[4] = {}, rd_fch[2] = {}, rd_qkv[2] = {}, ev_wte = nullptr, ev_end = nullptr;
    hipEvent_t fork[8] = {};
    int fork_next = 0;
    // MX FP8 forward products (caller memory from gpt2_mx_attach): E4M3 codes and
    // block scales of the forward weights, made from the bf16 copy whenever it has
    // changed, and one buffer for the quantized activation of the product at hand.
    // position encoding: learned wpe (default) or rotary (cos / sin table at `rope`)
    int pos_enc = GPT2_POS_LEARNED;
    size_t rope = 0;
    int gemm_format = GPT2_GEMM_BF16;
    char* mx = nullptr;
    size_t mx_bytes = 0;
    bool mx_stale = true;
    std::vector<size_t> mxq, mxs;  // [L * 4 + 1]: qkv, proj, fc, fc-proj per layer, then wte
    size_t mx_in_q = 0, mx_in_s = 0;    // codes of a C-wide product input (LayerNorm, attention)
    size_t mx_act_q = 0, mx_act_s = 0;  // codes of the 4C-wide GELU output
    // GPT2_GEMM_MXFP8_DX: codes of every forward weight's transpose W^T (blocks along
    // the layer's outputs) and of the upstream gradient of the input-gradient product
    // at hand
    std::vector<size_t> mxqT, mxsT;
    size_t mx_dy_q = 0, mx_dy_s = 0;    // up to B*T x vocab: the product at hand's upstream gradient
    size_t mx_dy2_q = 0, mx_dy2_s = 0;  // B*T x 4C: written by the GELU' product for the next one
    bool dlogits_codes = false;         // the last loss forward wrote the codes of d loss / d logits
};

// Incremental generation over an arena's parameters (bf16): the key/value cache holds
// every layer's q|k|v rows of each sequence, [L][batch][max_len][3C].
struct gpt2_gen {
    gpt2_arena* a;
    int batch, max_len, len;
    bool ready;
    char* base;
    size_t cache, res[3], atty, fchg, lnf, stats;
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// SwiGLU width of the Llama-style block: 8C/3 rounded up to a multiple of 64.
int64_t llama_hidden(int64_t C) { return 64 * ((C + 23) / 24); }

int64_t count_params(const gpt2_config& c, int64_t* o_layer, int64_t* o_wte, int64_t* o_wpe, int64_t* o_lnf,
                     int block = GPT2_BLOCK_GPT2) {
    // Layer-major order of the module tree (GPT-2 from scratch with torch, 总体架构):
    // wte, wpe, per block [ln_1 w,b; c_attn W,b; attn c_proj W,b; ln_2 w,b; c_fc W,b;
    // mlp c_proj W,b], ln_f w,b.  Weights are (out, in) row-major.  The Llama-style
    // block keeps the slots with the biases and shifts empty: [rms_1 w; qkv W; proj W;
    // rms_2 w; gate|up W (2H x C, gate and up rows interleaved); down W (C x H)], then
    // the final RMSNorm's w.
    const int64_t C = c.channels, H = llama_hidden(C);
    const int64_t gsz[P_N] = {C, C, 3 * C * C, 3 * C, C * C, C, C, C, 4 * C * C, 4 * C, 4 * C * C, C};
    const int64_t lsz[P_N] = {C, 0, 3 * C * C, 0, C * C, 0, C, 0, 2 * H * C, 0, C * H, 0};
    const int64_t* sz = block == GPT2_BLOCK_LLAMA ? lsz : gsz;
    int64_t o = 0;
    if (o_wte) *o_wte = o;
    o += (int64_t)c.vocab_size * C;
    if (o_wpe) *o_wpe = o;
    o += (int64_t)c.max_seq_len * C;
    for (int l = 0; l < c.num_layers; ++l)
        for (int i = 0; i < P_N; ++i) {
            if (o_layer) o_layer[l * P_N + i] = o;
            o += sz[i];
        }
    if (o_lnf) *o_lnf = o;
    return o + (block == GPT2_BLOCK_LLAMA ? 1 : 2) * C;
}

int validate(const gpt2_config* cfg, int B, int T, int dtype) {
    if (!cfg) return fail(GPT2_E_INVAL, "cfg is NULL");
    const gpt2_config& c = *cfg;
    if (c.channels <= 0 || c.num_heads <= 0 || c.num_layers <= 0 || c.vocab_size < 2 || c.max_seq_len <= 0)
        return fail(GPT2_E_INVAL, "non-positive model dimension");
    if (c.channels % c.num_heads) return fail(GPT2_E_INVAL, "channels must be a multiple of num_heads");
    if (c.channels % 8) return fail(GPT2_E_INVAL, "channels must be a multiple of 8");
    const int hs = c.channels / c.num_heads;
    if (hs != 16 && hs != 32 && hs != 64 && hs != 128)
        return fail(GPT2_E_INVAL, "head size (channels / num_heads) must be 16, 32, 64 or 128");
    if (c.channels > 2048) return fail(GPT2_E_INVAL, "channels must be <= 2048");
    if (B < 1 || T < 1 || T > c.max_seq_len) return fail(GPT2_E_INVAL, "need B >= 1 and 1 <= T <= max_seq_len");
    if ((int64_t)B * T > (1 << 30)) return fail(GPT2_E_INVAL, "B*T too large");
    // GEMM operands are addressed with 32-bit buffer offsets: the largest, the
    // logits [B*T, vocab rounded up to 64] in bf16 or fp32, must stay below 4 GiB.
    const int64_t vpad = ((int64_t)c.vocab_size + 63) / 64 * 64;
    if ((int64_t)B * T * vpad * (dtype == GPT2_BF16 ? 2 : 4) >= ((int64_t)1 << 32))
        return fail(GPT2_E_INVAL, "B*T*vocab too large for one arena (logits over 4 GiB)");
    if (dtype != GPT2_FP32 && dtype != GPT2_BF16) return fail(GPT2_E_INVAL, "dtype must be GPT2_FP32 or GPT2_BF16");
    return GPT2_OK;
}

// Computes every region's offset; returns the total byte size.
size_t layout(gpt2_arena& a) {
    const gpt2_config& c = a.cfg;
    const int64_t C = c.channels, L = c.num_layers, BT = (int64_t)a.B * a.T, NH = c.num_heads;
    const size_t es = a.act_size;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    a.params = take(a.nparams * 4);
    a.grads = take(a.nparams * 4);
    a.adam_m = take(a.nparams * 4);
    a.adam_v = take(a.nparams * 4);
    a.params16 = a.dtype == GPT2_BF16 ? take(a.nparams * 2) : 0;
    a.encoded = take(BT * C * es);
    a.la.resize(L);
    for (int l = 0; l < L; ++l) {
        LayerActs& x = a.la[l];
        x.ln1 = take(BT * C * es);
        x.ln1s = take(BT * 2 * 4);
        x.qkv = take(BT * 3 * C * es);
        x.atty = take(BT * C * es);
        x.lse = take(BT * NH * 4);
        x.res2 = take(BT * C * es);
        x.ln2 = take(BT * C * es);
        x.ln2s = take(BT * 2 * 4);
        x.fch = take(BT * a.F1 * es);
        x.fchg = take(BT * a.F2 * es);
        x.res3 = take(BT * C * es);
    }
    a.lnf = take(BT * C * es);
    a.lnfs = take(BT * 2 * 4);
    a.logits = take(BT * (int64_t)a.Vp * es);
    a.losses = take(BT * 4);
    a.loss = take(4);
    // backward scratch: a ring of four residual-gradient buffers and two of each of
    // dfch / dqkv, so the main stream never overwrites what the side stream reads
    for (int i = 0; i < 4; ++i) a.dres[i] = take(BT * C * es);
    a.dbuf = take(BT * C * es);
    for (int i = 0; i < 2; ++i) a.dqkv[i] = take(BT * 3 * C * es);
    for (int i = 0; i < 2; ++i) a.dfch[i] = take(BT * a.F1 * es);
    a.dh = a.block == GPT2_BLOCK_LLAMA ? take(BT * a.H * es) : 0;  // SwiGLU output gradient
    a.dsum = take(BT * NH * 8);  // per (row, head): {lse log2 e, D} for the head-size-64 kernels
    a.partial_floats = (size_t)512 * 2 * 4 * C;  // column-sum partials (<= 256 blocks x 4C)
    a.partial = take(a.partial_floats * 4);
    a.partial_side = take(a.partial_floats * 4);
    a.ws_floats = (size_t)16 * std::max<int64_t>(4 * C, 2 * a.H) * C;  // split-K partials of the largest dW, 16 splits
    a.ws = take(a.ws_floats * 4);
    // main stream's split-K partials: the tied-embedding dX ([B*T, C], K = vocab) in up to 4 splits
    a.ws_main_floats = (size_t)4 * BT * C;
    a.ws_main = take(a.ws_main_floats * 4);
    a.census = take((size_t)2 * a.cfg.vocab_size * 4);  // per token: first position, count (embedding backward)
    a.rope = take((size_t)a.cfg.max_seq_len * (a.hs / 2) * 8);  // rotary cos / sin table [P][hs / 2]
    return o;
}

template <class P>
P* at(const gpt2_arena* a, size_t off) {
    return (P*)(a->base + off);
}

int64_t round128(int64_t k) { return (k + 127) / 128 * 128; }

// Rows and k of the MX forward weights: index l * 4 + {0 qkv, 1 proj, 2 fc, 3 fc-proj}, then wte.
void mx_weight_shape(const gpt2_arena& a, int i, int64_t* rows, int64_t* k) {
    const int64_t C = a.cfg.channels;
    const int L = a.cfg.num_layers;
    if (i == 4 * L) { *rows = a.cfg.vocab_size; *k = C; return; }
    const int64_t r[4] = {3 * C, C, 4 * C, C}, kk[4] = {C, C, C, 4 * C};
    *rows = r[i % 4];
    *k = kk[i % 4];
}

// Offsets within the MX memory; returns its byte size.
size_t mx_layout(gpt2_arena& a) {
    const int L = a.cfg.num_layers;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    a.mxq.assign(4 * L + 1, 0);
    a.mxs.assign(4 * L + 1, 0);
    for (int i = 0; i <= 4 * L; ++i) {
        int64_t rows, k;
        mx_weight_shape(a, i, &rows, &k);
        a.mxq[i] = take((size_t)rows * round128(k));
        a.mxs[i] = take((size_t)rows * round128(k) / 32);
    }
    const int64_t BT = (int64_t)a.B * a.T, k1 = round128(a.cfg.channels), k4 = round128(4 * (int64_t)a.cfg.channels);
    a.mx_in_q = take((size_t)BT * k1);
    a.mx_in_s = take((size_t)BT * k1 / 32);
    a.mx_act_q = take((size_t)BT * k4);
    a.mx_act_s = take((size_t)BT * k4 / 32);
    // transposed weights: [k, rows rounded to 128] codes
    a.mxqT.assign(4 * L + 1, 0);
    a.mxsT.assign(4 * L + 1, 0);
    for (int i = 0; i <= 4 * L; ++i) {
        int64_t rows, k;
        mx_weight_shape(a, i, &rows, &k);
        a.mxqT[i] = take((size_t)k * round128(rows));
        a.mxsT[i] = take((size_t)k * round128(rows) / 32);
    }
    // upstream gradients: up to BT x V (the tied lm_head's), else BT x 4C
    const int64_t kdy = std::max(round128(a.cfg.vocab_size), k4);
    a.mx_dy_q = take((size_t)BT * kdy);
    a.mx_dy_s = take((size_t)BT * kdy / 32);
    a.mx_dy2_q = take((size_t)BT * k4);
    a.mx_dy2_s = take((size_t)BT * k4 / 32);
    return o;
}

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GPT2_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return GPT2_OK;
}

#define CHECK(expr, what)                                   \
    do {                                                    \
        int rc__ = hip_check((expr), what);                 \
        if (rc__ != GPT2_OK) return rc__;                   \
    } while (0)

int ensure_streams(gpt2_arena* a) {
    if (!a->side) {
        if (hipStreamCreateWithFlags(&a->side, hipStreamNonBlocking) != hipSuccess) {
            a->side = nullptr;
            return fail(GPT2_E_HIP, "cannot create the side stream");
        }
        a->side_owned = true;
    }
    if (a->events_ready) return GPT2_OK;
    auto mk = [](hipEvent_t* e) { return hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess; };
    bool ok = mk(&a->ev_wte) && mk(&a->ev_end);
    for (auto& e : a->rd_res) ok = ok && mk(&e);
    for (auto& e : a->rd_fch) ok = ok && mk(&e);
    for (auto& e : a->rd_qkv) ok = ok && mk(&e);
    for (auto& e : a->fork) ok = ok && mk(&e);
    a->events_ready = ok;
    return ok ? GPT2_OK : fail(GPT2_E_HIP, "cannot create events");
}

// `to` waits for everything enqueued on `from` so far.
int stream_wait(gpt2_arena* a, hipStream_t to, hipStream_t from) {
    hipEvent_t e = a->fork[a->fork_next];
    a->fork_next = (a->fork_next + 1) % 8;
    if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess)
        return fail(GPT2_E_HIP, "stream fork/join failed");
    return GPT2_OK;
}

void destroy_streams(gpt2_arena* a) {
    if (a->side && a->side_owned) hipStreamDestroy(a->side);
    a->side = nullptr;
    a->side_owned = false;
    if (!a->events_ready) return;
    auto rm = [](hipEvent_t& e) {
        if (e) hipEventDestroy(e);
        e = nullptr;
    };
    rm(a->ev_wte);
    rm(a->ev_end);
    for (auto& e : a->rd_res) rm(e);
    for (auto& e : a->rd_fch) rm(e);
    for (auto& e : a->rd_qkv) rm(e);
    for (auto& e : a->fork) rm(e);
    a->events_ready = false;
}

// AdamW hyper-parameters with the bias corrections of step t folded in.
struct AdamArgs {
    float lr, b1, b2, eps, wd, c1, c2;
};

AdamArgs adam_args(float lr, float b1, float b2, float eps, float wd, int32_t step) {
    return AdamArgs{lr, b1, b2, eps, wd, (float)(1.0 - pow((double)b1, (double)step)),
                    (float)(1.0 - pow((double)b2, (double)step))};
}

// AdamW over parameters [off, off + n) (offsets are multiples of 8: every tensor size is).
int adamw_range(gpt2_arena* a, const AdamArgs& o, int64_t off, int64_t n, hipStream_t s) {
    if (n <= 0) return GPT2_OK;
    bf16* p16 = a->dtype == GPT2_BF16 ? at<bf16>(a, a->params16) + off : nullptr;
    return hip_check(adamw(at<float>(a, a->params) + off, at<float>(a, a->grads) + off,
                           at<float>(a, a->adam_m) + off, at<float>(a, a->adam_v) + off, p16, n, o.lr, o.b1, o.b2,
                           o.eps, o.wd, o.c1, o.c2, s),
                     "adamw");
}

template <class T>
struct Model {
    gpt2_arena* a;
    hipStream_t s;
    int C, L, NH, V, Vp, B, S, BT, P;  // S: sequence length

    Model(gpt2_arena* ar, hipStream_t st) : Model(ar, st, ar->B, ar->T) {}
    // A forward pass over Be sequences of length Se in the arena's buffers (Be * Se <=
    // B * T): rows stay dense, [Be * Se, .], so every kernel sees an ordinary batch.
    Model(gpt2_arena* ar, hipStream_t st, int Be, int Se) : a(ar), s(st) {
        C = a->cfg.channels; L = a->cfg.num_layers; NH = a->cfg.num_heads; V = a->cfg.vocab_size;
        Vp = a->Vp; B = Be; S = Se; BT = B * S; P = a->cfg.max_seq_len;
    }
    // A forward pass over the Bg sequences b0 .. b0 + Bg - 1 of a batch (rows b0 S ..):
    // every per-row and per-sequence kernel sees only those rows, so the passes over two
    // such groups are independent and can run on two streams.
    int b0 = 0;
    bool side_group = false;  // runs on the side stream beside a main-stream group
    Model(gpt2_arena* ar, hipStream_t st, int Bg, int Se, int first, bool side = false) : Model(ar, st, Bg, Se) {
        b0 = first;
        side_group = side;
    }
    int64_t r0() const { return (int64_t)b0 * S; }
    T* arow(size_t off, int64_t width) const { return act(off) + r0() * width; }
    float* frow(size_t off, int64_t width) const { return f32(off) + r0() * width; }
    float* master(int64_t off) const { return at<float>(a, a->params) + off; }
    float* grad(int64_t off) const { return at<float>(a, a->grads) + off; }
    // GEMM weight operand: the bf16 copy in BF16 mode, the master in FP32 mode.
    const T* weight(int64_t off) const {
        if (a->dtype == GPT2_BF16) return (const T*)(at<bf16>(a, a->params16) + off);
        return (const T*)(at<float>(a, a->params) + off);
    }
    int64_t lp(int l, int i) const { return a->o_layer[l * P_N + i]; }
    T* act(size_t off) const { return at<T>(a, off); }
    float* f32(size_t off) const { return at<float>(a, off); }

    // Options of the bf16 / MX products' bias epilogue: the rotary turn of the q|k
    // columns and the SwiGLU output of a gate|up product (GemmArgs).
    struct EpiExtra {
        const float2* rope = nullptr;
        int period = 0, hs = 0, cols = 0;
        bf16* swiglu = nullptr;
        int64_t ld_swiglu = 0;
        const bf16* swiglu_gu = nullptr;  // backward: the saved (gate, up) pairs
    };
    static void apply_extra(GemmArgs& g, const EpiExtra& e) {
        g.rope = e.rope; g.rope_period = e.period; g.rope_hs = e.hs; g.rope_cols = e.cols;
        g.swiglu = e.swiglu; g.ld_swiglu = e.ld_swiglu; g.swiglu_gu = e.swiglu_gu;
    }

    int gemm_call(const void* A, int64_t lda, bool ak, const void* Bm, int64_t ldb, bool bk, void* Cm, int64_t ldc,
                  int M, int N, int K, int epi, const float* bias = nullptr, const void* R = nullptr,
                  void* C2 = nullptr, const EpiExtra& ex = EpiExtra{}) {
        GemmArgs g{};
        g.A = A; g.B = Bm; g.C = Cm; g.C2 = C2; g.R = R; g.bias = bias;
        g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc;
        apply_extra(g, ex);
        // main-stream products use their own split-K workspace (the side stream's is busy
        // during backward); the side group of a split forward pass splits no product
        CHECK(gemm<T>(g, ak, bk, epi, side_group ? nullptr : f32(a->ws_main), side_group ? 0 : a->ws_main_floats, s),
              "gemm");
        return GPT2_OK;
    }

    uint8_t* mxp(size_t off) const { return (uint8_t*)(a->mx + off); }
    bool rotary() const { return a->pos_enc == GPT2_POS_ROTARY; }
    bool llama() const { return a->block == GPT2_BLOCK_LLAMA; }
    // a bias / shift parameter of the block, or null for the Llama-style block (none)
    const float* pb(int64_t off) const { return llama() ? nullptr : master(off); }
    float* gb(int64_t off) const { return llama() ? nullptr : grad(off); }
    const float2* rope_tab() const { return at<float2>(a, a->rope); }
    float2* rope_tab_mut() const { return at<float2>(a, a->rope); }

    // MX codes and scales of the forward weights from the bf16 copy.
    int mx_refresh() {
        const bf16* w16 = at<bf16>(a, a->params16);
        // the codes of W and (for the input-gradient products) of W^T, from one read of W;
        // each of the four block weights in one launch over all layers (the layer-major
        // arena and the code layout put layer l + 1's copy at a fixed stride from layer l's)
        const bool dx = a->gemm_format == GPT2_GEMM_MXFP8_DX;
        static constexpr int which[4] = {P_QKVW, P_PROJW, P_FCW, P_FCPW};
        auto codes = [&](int i, int64_t off, int n, const MxWeightStrides& bs) {
            int64_t rows, k;
            mx_weight_shape(*a, i, &rows, &k);
            return hip_check(mx_weight_codes(w16 + off, k, (int)rows, (int)k, mxp(a->mxq[i]), round128(k),
                                             mxp(a->mxs[i]), dx ? mxp(a->mxqT[i]) : nullptr, round128(rows),
                                             dx ? mxp(a->mxsT[i]) : nullptr, s, n, bs),
                             "mx weights");
        };
        int rc;
        for (int t = 0; t < 4; ++t) {
            MxWeightStrides bs;
            bool uniform = L > 1;
            if (uniform) {
                bs.w = lp(1, which[t]) - lp(0, which[t]);
                bs.q = (int64_t)(a->mxq[t + 4] - a->mxq[t]);
                bs.sq = (int64_t)(a->mxs[t + 4] - a->mxs[t]);
                bs.qt = (int64_t)(a->mxqT[t + 4] - a->mxqT[t]);
                bs.sqt = (int64_t)(a->mxsT[t + 4] - a->mxsT[t]);
                // (the kernel's vector accesses need these alignments of the strides)
                uniform = bs.w % 8 == 0 && bs.q % 16 == 0 && bs.sq % 4 == 0 && bs.qt % 16 == 0 && bs.sqt % 4 == 0;
                for (int l = 1; l < L; ++l) {
                    const int i = 4 * l + t;
                    uniform = uniform && lp(l, which[t]) - lp(l - 1, which[t]) == bs.w &&
                              (int64_t)(a->mxq[i] - a->mxq[i - 4]) == bs.q &&
                              (int64_t)(a->mxs[i] - a->mxs[i - 4]) == bs.sq &&
                              (int64_t)(a->mxqT[i] - a->mxqT[i - 4]) == bs.qt &&
                              (int64_t)(a->mxsT[i] - a->mxsT[i - 4]) == bs.sqt;
                }
            }
            if (uniform) {  // every layer's copy of this weight in one launch
                if ((rc = codes(t, lp(0, which[t]), L, bs))) return rc;
            } else {
                for (int l = 0; l < L; ++l)
                    if ((rc = codes(4 * l + t, lp(l, which[t]), 1, MxWeightStrides{}))) return rc;
            }
        }
        if ((rc = codes(4 * L, a->o_wte, 1, MxWeightStrides{}))) return rc;
        a->mx_stale = false;
        return GPT2_OK;
    }

    bool mx_on() const {
        return sizeof(T) == 2 && (a->gemm_format == GPT2_GEMM_MXFP8 || a->gemm_format == GPT2_GEMM_MXFP8_DX);
    }
    bool mx_dx_on() const { return sizeof(T) == 2 && a->gemm_format == GPT2_GEMM_MXFP8_DX; }

    // MX codes of a product input: `codes` in buffer (q, s) with row stride ldq.
    struct MxBuf {
        uint8_t* q = nullptr;
        uint8_t* s = nullptr;
        int64_t ld = 0;
    };
    MxBuf mx_in() const { return mx_on() ? MxBuf{mxp(a->mx_in_q), mxp(a->mx_in_s), round128(C)} : MxBuf{}; }
    MxBuf mx_gelu() const {
        // the fc epilogue writes the GELU codes itself when 4C is a multiple of 128
        return mx_on() && (4 * C) % 128 == 0 ? MxBuf{mxp(a->mx_act_q), mxp(a->mx_act_s), round128(4 * C)} : MxBuf{};
    }

    // An input-gradient product dX = dY W (+ GELU' epilogue) with dY [BT, K] (row stride
    // ldy) and W [K, N] the weight of forward product `wi`: bf16, or with
    // GPT2_GEMM_MXFP8_DX dY's rows and W^T's rows (made at the forward pass's code
    // refresh) on MX codes.
    // codes of a C-wide upstream gradient written by the LayerNorm backward (the buffer of
    // the product at hand: each is consumed by the next input-gradient product on the
    // same stream before the next LayerNorm backward writes it again)
    MxBuf dy_codes() const {
        return mx_dx_on() && !llama() ? MxBuf{mxp(a->mx_dy_q), mxp(a->mx_dy_s), round128(C)} : MxBuf{};
    }

    // codes of the c_fc input gradient, written by the GELU' product's epilogue when 4C
    // is a multiple of 128 (its 16-thread groups then cover whole 128-column stages)
    MxBuf dfch_codes() const {
        return mx_dx_on() && !llama() && (4 * C) % 128 == 0
                   ? MxBuf{mxp(a->mx_dy2_q), mxp(a->mx_dy2_s), round128(4 * C)}
                   : MxBuf{};
    }

    // `codes`: dY's codes when its producer wrote them, else dY is quantized here;
    // `out_codes`: the GELU' product also writes the codes of its output.
    int dx_gemm(const T* dy, int64_t ldy, int K, int wi, int64_t w_off, void* out, int64_t ldc, int N, int epi,
                const void* R = nullptr, MxBuf codes = MxBuf{}, MxBuf out_codes = MxBuf{}) {
        if constexpr (sizeof(T) == 2) {
            if (mx_dx_on()) {
                const int64_t Kp = round128(K);
                if (!codes.q) {
                    codes = MxBuf{mxp(a->mx_dy_q), mxp(a->mx_dy_s), Kp};
                    CHECK(mx_quantize((const bf16*)dy, ldy, BT, K, codes.q, Kp, codes.s, s), "mx dY");
                }
                GemmArgs g{};
                g.A = codes.q; g.B = mxp(a->mxqT[wi]); g.C = out; g.R = R;
                g.M = BT; g.N = N; g.K = (int)Kp; g.lda = codes.ld; g.ldb = Kp; g.ldc = ldc;
                g.sa = codes.s; g.sb = mxp(a->mxsT[wi]); g.srows_a = BT; g.srows_b = N;
                g.q2 = out_codes.q; g.s2 = out_codes.s; g.ldq2 = out_codes.ld;
                CHECK(gemm_mx(g, epi, s), "mx gemm dX");
                return GPT2_OK;
            }
        }
        return gemm_call(dy, ldy, true, weight(w_off), N, false, out, ldc, BT, N, K, epi, nullptr, R);
    }

    // A forward product Y = X W^T (+ epilogue) with X [BT, K] dense and W (N, K) at
    // parameter offset w_off (MX index wi).  With the MX FP8 format the product runs on
    // MX codes: those of X already made by its producer (`in`), else quantized here
    // into the matching buffer; `out2` asks the GELU epilogue for its output's codes.
    int fwd_gemm(const T* X, int K, int64_t w_off, int wi, int N, T* Y, int64_t ldc, int epi,
                 const float* bias = nullptr, const void* R = nullptr, void* C2 = nullptr, MxBuf in = {},
                 MxBuf out2 = {}, const EpiExtra& ex = EpiExtra{}) {
        if constexpr (sizeof(T) == 2) {
            if (mx_on()) {
                const int64_t Kp = round128(K);
                if (!in.q) {
                    in = K == C ? MxBuf{mxp(a->mx_in_q), mxp(a->mx_in_s), Kp} : MxBuf{mxp(a->mx_act_q), mxp(a->mx_act_s), Kp};
                    CHECK(mx_quantize((const bf16*)X, K, BT, K, in.q, in.ld, in.s, s), "mx quantize");
                }
                GemmArgs g{};
                g.A = in.q; g.B = mxp(a->mxq[wi]); g.C = Y; g.C2 = C2; g.R = R; g.bias = bias;
                g.M = BT; g.N = N; g.K = (int)Kp; g.lda = in.ld; g.ldb = Kp; g.ldc = ldc;
                g.sa = in.s; g.sb = mxp(a->mxs[wi]); g.srows_a = BT; g.srows_b = N;
                g.q2 = out2.q; g.s2 = out2.s; g.ldq2 = out2.ld;
                apply_extra(g, ex);
                CHECK(gemm_mx(g, epi, s), "mx gemm");
                return GPT2_OK;
            }
        }
        return gemm_call(X, K, true, weight(w_off), K, true, Y, ldc, BT, N, K, epi, bias, R, C2, ex);
    }

    // The forward pass over this model's rows (all of them unless it is one group of
    // a split pass): activations, logits and, with targets, the per-row losses and their
    // gradient (scaled by dscale = 1 / (rows of the whole batch)).  inp / tgt point at the
    // whole batch.
    int forward_rows(const int32_t* inp, const int32_t* tgt, float dscale) {
        inp += r0();
        if (tgt) tgt += r0();
        CHECK(encoder_forward<T>(arow(a->encoded, C), inp, master(a->o_wte), rotary() ? nullptr : master(a->o_wpe),
                                 BT, S, C, s),
              "encoder");
        for (int l = 0; l < L; ++l) {
            const LayerActs& x = a->la[l];
            const T* xin = l == 0 ? arow(a->encoded, C) : arow(a->la[l - 1].res3, C);
            const MxBuf mi = mx_in(), mg = mx_gelu();
            CHECK(layernorm_forward<T>(arow(x.ln1, C), frow(x.ln1s, 2), xin, master(lp(l, P_LN1W)), pb(lp(l, P_LN1B)),
                                       BT, C, s, mi.q, mi.ld, mi.s, llama()),
                  "ln1");
            int rc;
            // qkv = ln1 W_qkv^T + b
            // with rotary positions the bf16 products turn q and k in their epilogue
            const bool fuse_rope = rotary() && sizeof(T) == 2;
            EpiExtra rx;
            if (fuse_rope) rx.rope = rope_tab(), rx.period = S, rx.hs = C / NH, rx.cols = 2 * C;
            if ((rc = fwd_gemm(arow(x.ln1, C), C, lp(l, P_QKVW), 4 * l, 3 * C, arow(x.qkv, 3 * C), 3 * C, EPI_BIAS,
                               pb(lp(l, P_QKVB)), nullptr, nullptr, mi, MxBuf{}, rx)))
                return rc;
            if (rotary() && !fuse_rope)  // turn q and k of every head for its position (in place)
                CHECK(rope_apply<T>(arow(x.qkv, 3 * C), 3 * C, BT, 2 * C, C / NH, S, 0, rope_tab(), false, s), "rope");
            // (with MX products the attention kernel writes its output's codes when it can)
            bool att_coded = false;
            CHECK(attention_forward<T>(arow(x.atty, C), f32(x.lse) + (int64_t)b0 * NH * S, arow(x.qkv, 3 * C), B, S,
                                       C, NH, s, mi.q, mi.ld, mi.s, &att_coded),
                  "attention");
            // res2 = xin + atty W_proj^T + b
            if ((rc = fwd_gemm(arow(x.atty, C), C, lp(l, P_PROJW), 4 * l + 1, C, arow(x.res2, C), C, EPI_BIAS_RES,
                               pb(lp(l, P_PROJB)), xin, nullptr, att_coded ? mi : MxBuf{})))
                return rc;
            CHECK(layernorm_forward<T>(arow(x.ln2, C), frow(x.ln2s, 2), arow(x.res2, C), master(lp(l, P_LN2W)),
                                       pb(lp(l, P_LN2B)), BT, C, s, mi.q, mi.ld, mi.s, llama()),
                  "ln2");
            if (llama()) {
                // (g | u) = ln2 W_gu^T (interleaved), h = silu(g) u, res3 = res2 + h W_down^T
                const int H = (int)a->H;
                EpiExtra sx;  // bf16: the product's epilogue writes h itself
                if (sizeof(T) == 2) sx.swiglu = (bf16*)arow(x.fchg, a->F2), sx.ld_swiglu = H;
                if ((rc = fwd_gemm(arow(x.ln2, C), C, lp(l, P_FCW), 4 * l + 2, 2 * H, arow(x.fch, a->F1), 2 * H,
                                   EPI_BIAS, nullptr, nullptr, nullptr, MxBuf{}, MxBuf{}, sx)))
                    return rc;
                if (sizeof(T) != 2)
                    CHECK(swiglu_forward<T>(arow(x.fchg, a->F2), arow(x.fch, a->F1), BT, H, s), "swiglu");
                if ((rc = fwd_gemm(arow(x.fchg, a->F2), H, lp(l, P_FCPW), 4 * l + 3, C, arow(x.res3, C), C,
                                   EPI_BIAS_RES, nullptr, arow(x.res2, C))))
                    return rc;
                continue;
            }
            // fch = ln2 W_fc^T + b, fchg = gelu(fch)
            if ((rc = fwd_gemm(arow(x.ln2, C), C, lp(l, P_FCW), 4 * l + 2, 4 * C, arow(x.fch, 4 * C), 4 * C,
                               EPI_BIAS_GELU, master(lp(l, P_FCB)), nullptr, arow(x.fchg, 4 * C), mi, mg)))
                return rc;
            // res3 = res2 + fchg W_fcproj^T + b
            if ((rc = fwd_gemm(arow(x.fchg, 4 * C), 4 * C, lp(l, P_FCPW), 4 * l + 3, C, arow(x.res3, C), C,
                               EPI_BIAS_RES, master(lp(l, P_FCPB)), arow(x.res2, C), nullptr, mg)))
                return rc;
        }
        const MxBuf mi = mx_in();
        CHECK(layernorm_forward<T>(arow(a->lnf, C), frow(a->lnfs, 2), arow(a->la[L - 1].res3, C), master(a->o_lnfw),
                                   pb(a->o_lnfb), BT, C, s, mi.q, mi.ld, mi.s, llama()),
              "lnf");
        // logits = lnf wte^T (tied lm_head, no bias); row stride Vp
        int rc;
        if ((rc = fwd_gemm(arow(a->lnf, C), C, a->o_wte, 4 * L, V, arow(a->logits, Vp), Vp, EPI_BIAS, nullptr,
                           nullptr, nullptr, mi)))
            return rc;
        if (tgt) {
            // the MX input-gradient format takes the codes of d loss / d logits from here
            const bool dz_codes = mx_dx_on() && r0() == 0 && BT == (int64_t)a->B * a->T;
            CHECK(crossentropy_fused<T>(arow(a->logits, Vp), f32(a->losses) + r0(), tgt, BT, V, Vp, dscale, s,
                                        dz_codes ? mxp(a->mx_dy_q) : nullptr, round128(V),
                                        dz_codes ? mxp(a->mx_dy_s) : nullptr),
                  "crossentropy");
            a->dlogits_codes = dz_codes;
        }
        return GPT2_OK;
    }

    // The forward pass.  Without MX products (whose quantized-input buffers are shared)
    // and outside the launch profiler, a batch of two or more sequences is split into two
    // groups whose passes run on the main and the side stream at once: each kernel of one
    // group then fills the units the other's leaves idle (a product with few output tiles,
    // an epilogue, a LayerNorm).  Every per-row and per-sequence result is the same as in
    // one pass, bit for bit.
    int forward(const int32_t* inp, const int32_t* tgt) {
        if ((a->gemm_format == GPT2_GEMM_MXFP8 || a->gemm_format == GPT2_GEMM_MXFP8_DX) && a->mx_stale) {
            int rc = mx_refresh();
            if (rc) return rc;
        }
        if (rotary() && !a->rope_ready) {  // Llama-style arenas: the table with the default base
            CHECK(rope_table(rope_tab_mut(), P, C / NH, 10000.0, s), "rope table");
            a->rope_ready = true;
        }
        const float dscale = 1.0f / BT;
        const bool split = B >= 2 && !mx_on() && !profiling() && b0 == 0;
        int rc;
        if (!split) {
            if ((rc = forward_rows(inp, tgt, dscale))) return rc;
        } else {
            if ((rc = ensure_streams(a))) return rc;
            const int B1 = B / 2;
            Model<T> m0(a, s, B1, S, 0), m1(a, a->side, B - B1, S, B1, true);
            if ((rc = stream_wait(a, a->side, s))) return rc;
            if ((rc = m1.forward_rows(inp, tgt, dscale))) return rc;
            if ((rc = m0.forward_rows(inp, tgt, dscale))) return rc;
            if ((rc = stream_wait(a, s, a->side))) return rc;
        }
        if (tgt) CHECK(mean_loss(f32(a->loss), f32(a->losses), BT, s), "mean loss");
        return GPT2_OK;
    }

    // Backward.  The main stream `s` runs the chain that feeds the next layer (dX
    // GEMMs, LayerNorm and attention backward); every parameter-gradient product
    // (weight GEMMs, bias column sums, the tied-embedding dW) runs on the side
    // stream, which forks after each producer and is joined at the end.
    // With `opt`, each layer's AdamW update runs on the side stream as soon as the
    // main stream is done with that layer (its last reader of the layer's weights is
    // the ln_1 backward), overlapping the backward pass of the layers below; the
    // embeddings and ln_f are updated after the join.
    int backward(const AdamArgs* opt = nullptr) {
        // The census arrays return to their idle state only when the embedding backward
        // runs; a pass that stops early (an error) leaves them holding its counts, so the
        // next pass must clear them first.
        struct Disarm {
            gpt2_arena* a;
            bool done = false;
            ~Disarm() { if (!done) a->census_armed = false; }
        } disarm{a};
        int rc = run_backward(opt);
        disarm.done = rc == GPT2_OK;
        return rc;
    }

    int run_backward(const AdamArgs* opt) {
        int rc;
        if (!a->census_armed) {  // first backward pass on this arena: arm the token census
            CHECK(token_census_reset(at<int>(a, a->census), at<int>(a, a->census) + V, V, s), "census reset");
            a->census_armed = true;
        }
        if ((rc = ensure_streams(a))) return rc;
        hipStream_t M = s, SD = profiling() ? s : a->side;
        T* dz = act(a->logits);
        T* dbuf = act(a->dbuf);
        float* part = f32(a->partial);
        float* part_side = f32(a->partial_side);
        // A buffer-release event not yet recorded in this pass was last recorded by an
        // earlier pass, whose side-stream work the main stream has already joined, so
        // waiting on it is skipped.  This keeps every wait inside the pass, which also
        // lets a caller capture the pass into a graph.
        hipEvent_t marked[16];
        int nmarked = 0;
        auto wait = [&](hipStream_t st, hipEvent_t e) -> int {
            bool live = false;
            for (int i = 0; i < nmarked; ++i) live |= marked[i] == e;
            if (!live) return GPT2_OK;
            return hipStreamWaitEvent(st, e, 0) == hipSuccess ? GPT2_OK : fail(GPT2_E_HIP, "hipStreamWaitEvent");
        };
        auto mark = [&](hipEvent_t e, hipStream_t st) -> int {
            bool seen = false;
            for (int i = 0; i < nmarked; ++i) seen |= marked[i] == e;
            if (!seen) marked[nmarked++] = e;
            return hipEventRecord(e, st) == hipSuccess ? GPT2_OK : fail(GPT2_E_HIP, "hipEventRecord");
        };
        // side-stream weight GEMM: dW = dY^T X (fp32, overwrites), db = column sums of dY
        // (bf16: taken inside the GEMM from its dY tiles; fp32: a separate reduction)
        auto side_dw = [&](const T* dy, int OC, const T* x, int IC, int64_t ow, int64_t ob) -> int {
            int r;
            constexpr bool fused_db = sizeof(T) == 2;
            GemmArgs g{};
            g.A = dy; g.B = x; g.C = grad(ow);
            g.M = OC; g.N = IC; g.K = BT; g.lda = OC; g.ldb = IC; g.ldc = IC;
            if (fused_db && ob >= 0) g.rowsum = grad(ob);
            if ((r = hip_check(gemm<T>(g, false, false, EPI_F32, f32(a->ws), a->ws_floats, SD), "gemm"))) return r;
            if (!fused_db && ob >= 0)
                return hip_check(bias_grad<T>(grad(ob), dy, BT, OC, OC, part_side, a->partial_floats, SD), "bias grad");
            return GPT2_OK;
        };

        // which token ids the batch holds (the embedding backward's census, and with `opt`
        // the split of wte's AdamW update into absent rows, early, and present rows, last)
        int* census_first = at<int>(a, a->census);
        int* census_count = census_first + V;
        CHECK(token_census(census_first, census_count, a->inputs, BT, M), "token census");
        // lm_head: dlnf = dz wte on the main stream; dwte = dz^T lnf (overwrites) on the side
        if ((rc = stream_wait(a, SD, M))) return rc;
        {
            GemmArgs g{};
            g.A = dz; g.B = act(a->lnf); g.C = grad(a->o_wte);
            g.M = V; g.N = C; g.K = BT; g.lda = Vp; g.ldb = C; g.ldc = C;
            CHECK(gemm<T>(g, false, false, EPI_F32, f32(a->ws), a->ws_floats, SD), "gemm");
        }
        if (!opt && (rc = mark(a->ev_wte, SD))) return rc;
        // (the tied lm_head's upstream gradient is zero in its padded columns V .. Vp - 1)
        if (mx_dx_on()) {
            const MxBuf dzc = a->dlogits_codes ? MxBuf{mxp(a->mx_dy_q), mxp(a->mx_dy_s), round128(V)} : MxBuf{};
            if ((rc = dx_gemm(dz, Vp, (int)Vp, 4 * L, a->o_wte, dbuf, C, C, EPI_BIAS, nullptr, dzc))) return rc;
        } else if ((rc = gemm_call(dz, Vp, true, weight(a->o_wte), C, false, dbuf, C, BT, C, V, EPI_BIAS))) {
            return rc;
        }
        a->dlogits_codes = false;
        AdamwRows wte_opt{};
        if (opt) {
            // rows of wte no token of the batch touches have their final gradient now: update
            // them on the side stream once the main stream's dX product has read wte
            wte_opt = AdamwRows{master(a->o_wte), at<float>(a, a->adam_m) + a->o_wte,
                                at<float>(a, a->adam_v) + a->o_wte,
                                a->dtype == GPT2_BF16 ? at<bf16>(a, a->params16) + a->o_wte : nullptr,
                                opt->lr, opt->b1, opt->b2, opt->eps, opt->wd, opt->c1, opt->c2};
            if ((rc = stream_wait(a, SD, M))) return rc;
            CHECK(adamw_rows_absent(wte_opt, grad(a->o_wte), census_count, V, C, SD), "adamw wte");
            if ((rc = mark(a->ev_wte, SD))) return rc;
        }
        int cur = 0;
        if ((rc = wait(M, a->rd_res[0]))) return rc;
        const MxBuf dyc = dy_codes();  // LayerNorm backward outputs feed the next dX product
        CHECK(layernorm_backward<T>(act(a->dres[0]), (const T*)nullptr, grad(a->o_lnfw), gb(a->o_lnfb), dbuf,
                                    act(a->la[L - 1].res3), f32(a->lnfs), master(a->o_lnfw), BT, C, part,
                                    a->partial_floats, M, llama(), dyc.q, dyc.ld, dyc.s),
              "lnf backward");
        const int64_t F1 = a->F1, F2 = a->F2;
        auto bias_off = [&](int64_t off) -> int64_t { return llama() ? -1 : off; };
        for (int l = L - 1; l >= 0; --l) {
            const LayerActs& x = a->la[l];
            const T* xin = l == 0 ? act(a->encoded) : act(a->la[l - 1].res3);
            const int i_in = cur, i_mid = (cur + 1) % 4, i_out = (cur + 2) % 4, p = l & 1;
            T* din = act(a->dres[i_in]);
            T* dmid = act(a->dres[i_mid]);
            T* dout = act(a->dres[i_out]);
            T* dfch = act(a->dfch[p]);
            T* dqkv = act(a->dqkv[p]);
            // mlp c_proj: side: dW = din^T fchg, db = colsum(din); main: dfch = (din W_fcproj) * gelu'(fch)
            if ((rc = stream_wait(a, SD, M))) return rc;
            if ((rc = side_dw(din, C, act(x.fchg), (int)F2, lp(l, P_FCPW), bias_off(lp(l, P_FCPB))))) return rc;
            if ((rc = mark(a->rd_res[i_in], SD))) return rc;
            if ((rc = wait(M, a->rd_fch[p]))) return rc;
            if (llama()) {  // dh = din W_down, then (dg | du) from silu(g) u
                const int H = (int)a->H;
                T* dh = act(a->dh);
                EpiExtra bx;  // bf16: the dX product's epilogue writes (dg | du) itself
                if (sizeof(T) == 2) bx.swiglu = (bf16*)dfch, bx.ld_swiglu = H, bx.swiglu_gu = (const bf16*)act(x.fch);
                if ((rc = gemm_call(din, C, true, weight(lp(l, P_FCPW)), H, false, dh, H, BT, H, C, EPI_BIAS, nullptr,
                                    nullptr, nullptr, bx)))
                    return rc;
                if (sizeof(T) != 2) CHECK(swiglu_backward<T>(dfch, dh, act(x.fch), BT, H, M), "swiglu backward");
            } else if ((rc = dx_gemm(din, C, C, 4 * l + 3, lp(l, P_FCPW), dfch, 4 * C, 4 * C, EPI_GELU_BWD,
                                     act(x.fch), dyc, dfch_codes()))) {
                return rc;
            }
            // c_fc: side: dW = dfch^T ln2, db = colsum(dfch); main: dln2 = dfch W_fc
            if ((rc = stream_wait(a, SD, M))) return rc;
            if ((rc = side_dw(dfch, (int)F1, act(x.ln2), C, lp(l, P_FCW), bias_off(lp(l, P_FCB))))) return rc;
            if ((rc = mark(a->rd_fch[p], SD))) return rc;
            if ((rc = dx_gemm(dfch, F1, (int)F1, 4 * l + 2, lp(l, P_FCW), dbuf, C, C, EPI_BIAS, nullptr,
                              dfch_codes())))
                return rc;
            // ln_2: dmid = din + LN backward
            if ((rc = wait(M, a->rd_res[i_mid]))) return rc;
            CHECK(layernorm_backward<T>(dmid, din, grad(lp(l, P_LN2W)), gb(lp(l, P_LN2B)), dbuf, act(x.res2),
                                        f32(x.ln2s), master(lp(l, P_LN2W)), BT, C, part, a->partial_floats, M,
                                        llama(), dyc.q, dyc.ld, dyc.s),
                  "ln2 backward");
            // attn c_proj: side: dW = dmid^T atty, db; main: datty = dmid W_proj
            if ((rc = stream_wait(a, SD, M))) return rc;
            if ((rc = side_dw(dmid, C, act(x.atty), C, lp(l, P_PROJW), bias_off(lp(l, P_PROJB))))) return rc;
            if ((rc = mark(a->rd_res[i_mid], SD))) return rc;
            if ((rc = dx_gemm(dmid, C, C, 4 * l + 1, lp(l, P_PROJW), dbuf, C, C, EPI_BIAS, nullptr, dyc))) return rc;
            // attention
            if ((rc = wait(M, a->rd_qkv[p]))) return rc;
            CHECK(attention_backward<T>(dqkv, f32(a->dsum), dbuf, act(x.atty), act(x.qkv), f32(x.lse), B, S, C, NH, M),
                  "attention backward");
            if (rotary())  // gradients of the turned q, k -> of the qkv product's output
                CHECK(rope_apply<T>(dqkv, 3 * C, BT, 2 * C, C / NH, S, 0, rope_tab(), true, M), "rope backward");
            // c_attn: side: dW = dqkv^T ln1, db; main: dln1 = dqkv W_qkv
            if ((rc = stream_wait(a, SD, M))) return rc;
            if ((rc = side_dw(dqkv, 3 * C, act(x.ln1), C, lp(l, P_QKVW), bias_off(lp(l, P_QKVB))))) return rc;
            if ((rc = mark(a->rd_qkv[p], SD))) return rc;
            if ((rc = dx_gemm(dqkv, 3 * C, 3 * C, 4 * l, lp(l, P_QKVW), dbuf, C, C, EPI_BIAS))) return rc;
            // ln_1: dout = dmid + LN backward (= d xin)
            if ((rc = wait(M, a->rd_res[i_out]))) return rc;
            // (layer 0's output feeds no product: no codes)
            const MxBuf dyc1 = l > 0 ? dyc : MxBuf{};
            CHECK(layernorm_backward<T>(dout, dmid, grad(lp(l, P_LN1W)), gb(lp(l, P_LN1B)), dbuf, xin, f32(x.ln1s),
                                        master(lp(l, P_LN1W)), BT, C, part, a->partial_floats, M, llama(), dyc1.q,
                                        dyc1.ld, dyc1.s),
                  "ln1 backward");
            cur = i_out;
            if (opt) {  // layer l's gradients are complete and its weights no longer read
                if ((rc = stream_wait(a, SD, M))) return rc;
                const int64_t beg = lp(l, 0), end = l + 1 < L ? lp(l + 1, 0) : a->o_lnfw;
                if ((rc = adamw_range(a, *opt, beg, end - beg, SD))) return rc;
            }
        }
        // embedding: dwte += scatter (after the side stream's lm_head dW), dwpe
        if ((rc = wait(M, a->ev_wte))) return rc;
        // (with `opt` the present rows of wte get their AdamW update as their gradient completes)
        CHECK(encoder_backward<T>(grad(a->o_wte), grad(a->o_wpe), act(a->dres[cur]), a->inputs, B, S, P, C,
                                  census_first, census_count, M, !rotary(), wte_opt),
              "encoder backward");
        // join: everything the side stream enqueued finishes before later main-stream work
        if ((rc = mark(a->ev_end, SD))) return rc;
        if ((rc = wait(M, a->ev_end))) return rc;
        if (opt) {
            if ((rc = adamw_range(a, *opt, a->o_wpe, lp(0, 0) - a->o_wpe, M))) return rc;  // wpe (wte: above)
            if ((rc = adamw_range(a, *opt, a->o_lnfw, a->nparams - a->o_lnfw, M))) return rc;  // ln_f
        }
        return GPT2_OK;
    }
};

}  // namespace

namespace {

// Row buffers of one decode step, as byte offsets from `base`: the residual rows (three
// in rotation), the attention output, the GELU output, the final LayerNorm output and
// its statistics.
struct DecodeRows {
    char* base;
    size_t res[3], atty, fchg, lnf, stats;
};

DecodeRows decode_rows_layout(int batch, int C, char* base, size_t* bytes) {
    DecodeRows r{};
    r.base = base;
    size_t o = 0;
    auto take = [&](size_t n) {
        const size_t at = o;
        o = align_up(o + n);
        return at;
    };
    const size_t Bg = batch, Cs = C;
    for (auto& x : r.res) x = take(Bg * Cs * 2);
    r.atty = take(Bg * Cs * 2);
    r.fchg = take(Bg * 4 * Cs * 2);
    r.lnf = take(Bg * Cs * 2);
    r.stats = take(Bg * 2 * 4);
    if (bytes) *bytes = o;
    return r;
}

// Static decode scratch of gpt2_gen_decode_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): each device's address is looked up once with
// hipGetSymbolAddress and kept here.
constexpr size_t kDecodeScratchBytes = 384 * 1024;
__device__ __align__(256) char scratch[kDecodeScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the calling thread's current device (looked up on first use).
int decode_scratch_ptr(char** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GPT2_E_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(GPT2_E_INVAL, "device index out of range for the static scratch");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(GPT2_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = (char*)p;
    }
    *out = g_scratch_ptr[dev];
    return GPT2_OK;
}

int decode_check(gpt2_gen* g, const int32_t* d_tokens, float* d_logits) {
    if (!g || !d_tokens || !d_logits) return fail(GPT2_E_INVAL, "generation state, tokens and logits are required");
    if (!g->ready) return fail(GPT2_E_STATE, "decode needs a preceding prefill");
    if (g->len >= g->max_len) return fail(GPT2_E_SIZE, "the cache is full (length == max_len)");
    return GPT2_OK;
}

// One decode step with the step's row buffers at `rows` (the generation state's own
// memory, or the static scratch of gpt2_gen_decode_noalloc); arguments already checked.
int decode_step(gpt2_gen* g, const int32_t* d_tokens, float* d_logits, hipStream_t s, const DecodeRows& rows) {
    gpt2_arena* a = g->a;
    const int C = a->cfg.channels, L = a->cfg.num_layers, NH = a->cfg.num_heads, V = a->cfg.vocab_size;
    const int Bg = g->batch, t = g->len;
    const int64_t C3 = 3 * (int64_t)C, row = (int64_t)g->max_len * C3;
    auto buf = [&](size_t off) { return (bf16*)(g->base + off); };          // the key/value cache
    auto rb = [&](size_t off) { return (bf16*)(rows.base + off); };          // the step's rows
    const float* master = at<float>(a, a->params);
    const bf16* w16 = at<bf16>(a, a->params16);
    auto lp = [&](int l, int i) { return a->o_layer[l * P_N + i]; };
    // x' = LayerNorm(x) with the gains / shifts at `ln` (if >= 0), then x' W^T
    auto skinny = [&](const bf16* x, int64_t ldx, int64_t ln, int64_t woff, int N, int K, void* Cout, int64_t ldc,
                      bf16* C2, const bf16* R, const float* bias, int epi) -> int {
        SkinnyArgs k{};
        k.x = x; k.ldx = ldx; k.W = w16 + woff; k.ldw = K; k.C = Cout; k.ldc = ldc; k.C2 = C2;
        k.R = R; k.ldr = C; k.bias = bias; k.M = Bg; k.N = N; k.K = K;
        if (ln >= 0) {
            k.ln_w = master + ln;
            k.ln_b = master + ln + K;
        }
        return hip_check(skinny_gemm(k, epi, s), "skinny gemm");
    };
    int rc;
    // x = wte[token] + wpe[t] for the one new row of every sequence
    const bool rot = a->pos_enc == GPT2_POS_ROTARY;
    CHECK(encoder_forward<bf16>(rb(rows.res[0]), d_tokens, master + a->o_wte, rot ? nullptr : master + a->o_wpe, Bg, 1,
                                C, s, t),
          "encoder");
    int cur = 0;
    for (int l = 0; l < L; ++l) {
        bf16* xin = rb(rows.res[cur]);
        bf16* res2 = rb(rows.res[(cur + 1) % 3]);
        bf16* res3 = rb(rows.res[(cur + 2) % 3]);
        bf16* cache = buf(g->cache) + (int64_t)l * Bg * row;
        // ln_1, then q|k|v of the new rows straight into cache row t of each sequence
        if ((rc = skinny(xin, C, lp(l, P_LN1W), lp(l, P_QKVW), 3 * C, C, cache + (int64_t)t * C3, row, nullptr,
                         nullptr, master + lp(l, P_QKVB), EPI_BIAS)))
            return rc;
        if (rot)  // the new rows' q and k, all at position t
            CHECK(rope_apply<bf16>(cache + (int64_t)t * C3, row, Bg, 2 * C, C / NH, 1, t, at<float2>(a, a->rope), false,
                                   s),
                  "rope");
        CHECK(attention_decode(rb(rows.atty), cache, Bg, t + 1, C, NH, row, s), "attention");
        if ((rc = skinny(rb(rows.atty), C, -1, lp(l, P_PROJW), C, C, res2, C, nullptr, xin, master + lp(l, P_PROJB),
                         EPI_BIAS_RES)))
            return rc;
        // ln_2, c_fc + GELU
        if ((rc = skinny(res2, C, lp(l, P_LN2W), lp(l, P_FCW), 4 * C, C, nullptr, 4 * C, rb(rows.fchg), nullptr,
                         master + lp(l, P_FCB), EPI_BIAS_GELU)))
            return rc;
        if ((rc = skinny(rb(rows.fchg), 4 * C, -1, lp(l, P_FCPW), C, 4 * C, res3, C, nullptr, res2,
                         master + lp(l, P_FCPB), EPI_BIAS_RES)))
            return rc;
        cur = (cur + 2) % 3;
    }
    // ln_f on its own (the lm_head product has thousands of blocks), then the next-token
    // logits (tied lm_head), fp32 [batch, V]
    CHECK(layernorm_forward<bf16>(rb(rows.lnf), (float*)(rows.base + rows.stats), rb(rows.res[cur]), master + a->o_lnfw,
                                  master + a->o_lnfb, Bg, C, s),
          "lnf");
    if ((rc = skinny(rb(rows.lnf), C, -1, a->o_wte, V, C, d_logits, V, nullptr, nullptr, nullptr, EPI_F32))) return rc;
    g->len = t + 1;
    return GPT2_OK;
}


}  // namespace

extern "C" {

const char* gpt2_last_error(void) { return g_error.c_str(); }

int64_t gpt2_num_parameters(const gpt2_config* cfg) {
    if (!cfg) return -1;
    return count_params(*cfg, nullptr, nullptr, nullptr, nullptr);
}

int64_t gpt2_num_parameters_block(const gpt2_config* cfg, int32_t block) {
    if (!cfg || (block != GPT2_BLOCK_GPT2 && block != GPT2_BLOCK_LLAMA)) return -1;
    return count_params(*cfg, nullptr, nullptr, nullptr, nullptr, block);
}

int gpt2_alloc_arena(const gpt2_config* cfg, int32_t B, int32_t T, int32_t dtype, void* device_base,
                     size_t device_bytes, size_t* required_bytes, gpt2_arena** out) {
    return gpt2_alloc_arena_block(cfg, GPT2_BLOCK_GPT2, B, T, dtype, device_base, device_bytes, required_bytes, out);
}

int gpt2_alloc_arena_block(const gpt2_config* cfg, int32_t block, int32_t B, int32_t T, int32_t dtype,
                           void* device_base, size_t device_bytes, size_t* required_bytes, gpt2_arena** out) {
    if (out) *out = nullptr;
    int rc = validate(cfg, B, T, dtype);
    if (rc) return rc;
    if (block != GPT2_BLOCK_GPT2 && block != GPT2_BLOCK_LLAMA) return fail(GPT2_E_INVAL, "unknown block type");
    gpt2_arena* a = new (std::nothrow) gpt2_arena();
    if (!a) return fail(GPT2_E_INVAL, "host allocation failed");
    a->cfg = *cfg;
    a->B = B;
    a->T = T;
    a->dtype = dtype;
    a->Vp = (cfg->vocab_size + 63) / 64 * 64;
    a->hs = cfg->channels / cfg->num_heads;
    a->act_size = dtype == GPT2_BF16 ? 2 : 4;
    a->block = block;
    a->H = llama_hidden(cfg->channels);
    a->F1 = block == GPT2_BLOCK_LLAMA ? 2 * a->H : 4 * (int64_t)cfg->channels;
    a->F2 = block == GPT2_BLOCK_LLAMA ? a->H : 4 * (int64_t)cfg->channels;
    if (block == GPT2_BLOCK_LLAMA) a->pos_enc = GPT2_POS_ROTARY;  // table built by the first forward pass
    a->o_layer.resize((size_t)cfg->num_layers * P_N);
    int64_t o_lnf = 0;
    a->nparams = count_params(*cfg, a->o_layer.data(), &a->o_wte, &a->o_wpe, &o_lnf, block);
    a->o_lnfw = o_lnf;
    a->o_lnfb = o_lnf + cfg->channels;  // (Llama-style: no final shift; unused)
    size_t need = layout(*a);
    if (required_bytes) *required_bytes = need;
    if (!device_base) {
        delete a;
        return GPT2_OK;
    }
    if ((uintptr_t)device_base % kAlign) {
        delete a;
        return fail(GPT2_E_ALIGN, "device_base must be 256-byte aligned");
    }
    if (device_bytes < need) {
        delete a;
        return fail(GPT2_E_SIZE, "device buffer too small: need " + std::to_string(need) + " bytes");
    }
    a->base = (char*)device_base;
    a->bytes = device_bytes;
    a->loss_ready = false;
    a->inputs = nullptr;
    if (!out) {
        delete a;
        return fail(GPT2_E_INVAL, "out is NULL");
    }
    *out = a;
    return GPT2_OK;
}

int gpt2_free_arena(gpt2_arena* a) {
    if (a) destroy_streams(a);
    delete a;
    return GPT2_OK;
}

int gpt2_sync_weights(gpt2_arena* a, void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    a->mx_stale = true;
    if (a->dtype == GPT2_BF16)
        return hip_check(cast_bf16(at<bf16>(a, a->params16), at<float>(a, a->params), a->nparams, (hipStream_t)stream),
                         "cast");
    return GPT2_OK;
}

int gpt2_set_side_stream(gpt2_arena* a, void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (a->side && a->side_owned) {
        // work already enqueued there must not be cut off by the destroy
        if (hipStreamSynchronize(a->side) != hipSuccess) return fail(GPT2_E_HIP, "hipStreamSynchronize");
        hipStreamDestroy(a->side);
    }
    a->side = (hipStream_t)stream;
    a->side_owned = false;
    return GPT2_OK;
}

int gpt2_forward(gpt2_arena* a, const int32_t* d_inputs, const int32_t* d_targets, void* stream) {
    if (!a || !d_inputs) return fail(GPT2_E_INVAL, "arena and inputs are required");
    a->loss_ready = false;
    a->inputs = d_inputs;
    int rc = a->dtype == GPT2_BF16 ? Model<bf16>(a, (hipStream_t)stream).forward(d_inputs, d_targets)
                                   : Model<float>(a, (hipStream_t)stream).forward(d_inputs, d_targets);
    if (rc == GPT2_OK && d_targets) a->loss_ready = true;
    return rc;
}

int gpt2_eval_loss(gpt2_arena* a, const int32_t* d_inputs, const int32_t* d_targets, int32_t num_batches,
                   float* d_loss, void* stream) {
    if (!a || !d_inputs || !d_targets || !d_loss) return fail(GPT2_E_INVAL, "arena, tokens and loss are required");
    if (num_batches < 1) return fail(GPT2_E_INVAL, "num_batches must be >= 1");
    const int64_t bt = (int64_t)a->B * a->T;
    const float scale = 1.0f / (float)num_batches;
    hipStream_t s = (hipStream_t)stream;
    for (int32_t i = 0; i < num_batches; ++i) {
        int rc = gpt2_forward(a, d_inputs + i * bt, d_targets + i * bt, stream);
        if (rc) return rc;
        if ((rc = hip_check(scaled_accumulate(d_loss, at<float>(a, a->loss), scale, i == 0, s), "loss mean")))
            return rc;
    }
    a->loss_ready = false;  // the logits hold the last batch's gradient, not a step's
    a->inputs = nullptr;
    return GPT2_OK;
}

int gpt2_backward(gpt2_arena* a, void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (!a->loss_ready) return fail(GPT2_E_STATE, "backward needs a preceding forward with targets");
    a->loss_ready = false;  // dlogits are consumed
    return a->dtype == GPT2_BF16 ? Model<bf16>(a, (hipStream_t)stream).backward()
                                 : Model<float>(a, (hipStream_t)stream).backward();
}

int gpt2_adamw_step(gpt2_arena* a, float lr, float beta1, float beta2, float eps, float weight_decay, int32_t step,
                    void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (step < 1) return fail(GPT2_E_INVAL, "step must be >= 1");
    a->mx_stale = true;
    return adamw_range(a, adam_args(lr, beta1, beta2, eps, weight_decay, step), 0, a->nparams, (hipStream_t)stream);
}

int gpt2_backward_adamw(gpt2_arena* a, float lr, float beta1, float beta2, float eps, float weight_decay,
                        int32_t step, void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (step < 1) return fail(GPT2_E_INVAL, "step must be >= 1");
    if (!a->loss_ready) return fail(GPT2_E_STATE, "backward needs a preceding forward with targets");
    a->loss_ready = false;
    a->mx_stale = true;
    const AdamArgs o = adam_args(lr, beta1, beta2, eps, weight_decay, step);
    return a->dtype == GPT2_BF16 ? Model<bf16>(a, (hipStream_t)stream).backward(&o)
                                 : Model<float>(a, (hipStream_t)stream).backward(&o);
}

int gpt2_set_position_encoding(gpt2_arena* a, int32_t mode, float base, void* stream) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (mode == GPT2_POS_LEARNED) {
        if (a->block == GPT2_BLOCK_LLAMA) return fail(GPT2_E_INVAL, "the Llama-style block uses rotary positions");
        a->pos_enc = mode;
        return GPT2_OK;
    }
    if (mode != GPT2_POS_ROTARY) return fail(GPT2_E_INVAL, "unknown position encoding");
    if (!(base > 1.f) || !std::isfinite(base)) return fail(GPT2_E_INVAL, "rotary base must be finite and > 1");
    int rc = hip_check(rope_table(at<float2>(a, a->rope), a->cfg.max_seq_len, a->hs, (double)base, (hipStream_t)stream),
                       "rope table");
    if (rc) return rc;
    a->pos_enc = mode;
    a->rope_ready = true;
    return GPT2_OK;
}

int gpt2_mx_attach(gpt2_arena* a, void* device_base, size_t device_bytes, size_t* required_bytes) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (a->block != GPT2_BLOCK_GPT2) return fail(GPT2_E_INVAL, "MX products are built for the GPT-2 block");
    if (a->dtype != GPT2_BF16) return fail(GPT2_E_INVAL, "MX FP8 products need a bf16 arena");
    const size_t need = mx_layout(*a);
    if (required_bytes) *required_bytes = need;
    if (!device_base) return GPT2_OK;
    if ((uintptr_t)device_base % kAlign) return fail(GPT2_E_ALIGN, "device_base must be 256-byte aligned");
    if (device_bytes < need) return fail(GPT2_E_SIZE, "MX buffer too small: need " + std::to_string(need) + " bytes");
    a->mx = (char*)device_base;
    a->mx_bytes = device_bytes;
    a->mx_stale = true;
    return GPT2_OK;
}

int gpt2_set_gemm_format(gpt2_arena* a, int32_t format) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (format == GPT2_GEMM_BF16) {
        a->gemm_format = format;
        return GPT2_OK;
    }
    if (format != GPT2_GEMM_MXFP8 && format != GPT2_GEMM_MXFP8_DX) return fail(GPT2_E_INVAL, "unknown GEMM format");
    if (a->block != GPT2_BLOCK_GPT2) return fail(GPT2_E_INVAL, "MX products are built for the GPT-2 block");
    if (!a->mx) return fail(GPT2_E_STATE, "the MX formats need memory from gpt2_mx_attach");
    if (a->dtype != GPT2_BF16) return fail(GPT2_E_INVAL, "the MX formats are built for bf16 arenas");
    a->gemm_format = format;
    a->mx_stale = true;
    return GPT2_OK;
}

int gpt2_mx_buffer(const gpt2_arena* a, int32_t which, size_t* codes_offset, size_t* scales_offset, int64_t* rows,
                   int64_t* ld) {
    if (!a || !codes_offset || !scales_offset || !rows || !ld) return fail(GPT2_E_INVAL, "NULL argument");
    if (!a->mx) return fail(GPT2_E_STATE, "no MX memory attached");
    const int64_t C = a->cfg.channels;
    *rows = (int64_t)a->B * a->T;
    if (which == GPT2_MX_BUF_INPUT) {
        *codes_offset = a->mx_in_q;
        *scales_offset = a->mx_in_s;
        *ld = round128(C);
    } else if (which == GPT2_MX_BUF_GELU) {
        *codes_offset = a->mx_act_q;
        *scales_offset = a->mx_act_s;
        *ld = round128(4 * C);
    } else if (which == GPT2_MX_BUF_DY) {
        if (a->gemm_format != GPT2_GEMM_MXFP8_DX) return fail(GPT2_E_STATE, "the dY buffer exists in the MX dX format only");
        *codes_offset = a->mx_dy_q;
        *scales_offset = a->mx_dy_s;
        *ld = round128(a->cfg.vocab_size);
    } else {
        return fail(GPT2_E_INVAL, "unknown MX buffer");
    }
    return GPT2_OK;
}

int gpt2_mx_weight_codes(const gpt2_arena* a, int32_t index, int32_t transposed, size_t* codes_offset,
                         size_t* scales_offset, int64_t* rows, int64_t* ld) {
    if (!a || !codes_offset || !scales_offset || !rows || !ld) return fail(GPT2_E_INVAL, "NULL argument");
    if (!a->mx) return fail(GPT2_E_STATE, "no MX memory attached");
    if (index < 0 || index > 4 * a->cfg.num_layers) return fail(GPT2_E_INVAL, "weight index out of range");
    int64_t r, k;
    mx_weight_shape(*a, index, &r, &k);
    if (transposed) {
        *codes_offset = a->mxqT[index];
        *scales_offset = a->mxsT[index];
        *rows = k;
        *ld = round128(r);
    } else {
        *codes_offset = a->mxq[index];
        *scales_offset = a->mxs[index];
        *rows = r;
        *ld = round128(k);
    }
    return GPT2_OK;
}

int gpt2_mx_quantize(const void* d_x, int64_t ldx, int32_t rows, int32_t K, void* d_codes, int64_t ldq,
                     void* d_scales, void* stream) {
    if (rows < 0 || K < 0) return fail(GPT2_E_INVAL, "negative size");
    if (rows == 0 || K == 0) return GPT2_OK;
    if (!d_x || !d_codes || !d_scales) return fail(GPT2_E_INVAL, "x, codes and scales are required");
    if (K % 8 || ldx < K || ldx % 8 || ldq < round128(K) || ldq % 16)
        return fail(GPT2_E_INVAL, "need K % 8 == 0, ldx >= K (a multiple of 8), ldq >= K rounded up to 128 (a multiple of 16)");
    return hip_check(mx_quantize((const bf16*)d_x, ldx, rows, K, (uint8_t*)d_codes, ldq, (uint8_t*)d_scales,
                                 (hipStream_t)stream),
                     "mx_quantize");
}

int gpt2_mx_gemm(const void* d_qa, const void* d_sa, int64_t lda, const void* d_qb, const void* d_sb, int64_t ldb,
                 void* d_c, int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t epilogue, const float* d_bias,
                 const void* d_residual, void* d_c2, void* stream) {
    if (M < 0 || N < 0 || K < 0) return fail(GPT2_E_INVAL, "negative size");
    if (M == 0 || N == 0) return GPT2_OK;
    if (K == 0 || K % 128) return fail(GPT2_E_INVAL, "K must be a positive multiple of 128 (zero-padded codes)");
    if (lda < K || ldb < K || lda % 16 || ldb % 16 || ldc < N || ldc % 8)
        return fail(GPT2_E_INVAL, "need lda, ldb >= K (multiples of 16) and ldc >= N (a multiple of 8)");
    if (!d_qa || !d_sa || !d_qb || !d_sb || !d_c) return fail(GPT2_E_INVAL, "operands and output are required");
    int epi;
    switch (epilogue) {
        case GPT2_EPI_BIAS: epi = EPI_BIAS; break;
        case GPT2_EPI_BIAS_RES: epi = EPI_BIAS_RES; break;
        case GPT2_EPI_BIAS_GELU: epi = EPI_BIAS_GELU; break;
        case GPT2_EPI_GELU_BWD: epi = EPI_GELU_BWD; break;
        default: return fail(GPT2_E_INVAL, "unknown epilogue");
    }
    if (epi == EPI_BIAS_RES && !d_residual) return fail(GPT2_E_INVAL, "GPT2_EPI_BIAS_RES needs the residual");
    if (epi == EPI_GELU_BWD && (!d_residual || d_bias))
        return fail(GPT2_E_INVAL, "GPT2_EPI_GELU_BWD needs the GELU input and takes no bias");
    if (epi == EPI_BIAS_GELU && !d_c2) return fail(GPT2_E_INVAL, "GPT2_EPI_BIAS_GELU needs the second output");
    if ((int64_t)M * lda >= ((int64_t)1 << 32) || (int64_t)N * ldb >= ((int64_t)1 << 32))
        return fail(GPT2_E_SIZE, "operands over 4 GiB");
    GemmArgs g{};
    g.A = d_qa; g.B = d_qb; g.C = d_c; g.C2 = d_c2; g.R = d_residual; g.bias = d_bias;
    g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.sa = (const uint8_t*)d_sa; g.sb = (const uint8_t*)d_sb; g.srows_a = M; g.srows_b = N;
    return hip_check(gemm_mx(g, epi, (hipStream_t)stream), "mx gemm");
}

int gpt2_tensor_info(const gpt2_arena* a, int32_t id, int32_t layer, size_t* byte_offset, int64_t* rows,
                     int64_t* cols, int64_t* row_stride, int32_t* dtype) {
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    const int64_t BT = (int64_t)a->B * a->T, C = a->cfg.channels, NH = a->cfg.num_heads;
    const int act = a->dtype;
    size_t off = 0;
    int64_t r = 0, c = 0, ld = -1;
    int32_t dt = GPT2_FP32;
    const bool per_layer = id >= GPT2_T_LN1;
    if (per_layer && (layer < 0 || layer >= a->cfg.num_layers)) return fail(GPT2_E_INVAL, "layer out of range");
    const LayerActs* x = per_layer ? &a->la[layer] : nullptr;
    switch (id) {
        case GPT2_T_PARAMS: off = a->params; r = 1; c = a->nparams; break;
        case GPT2_T_GRADS: off = a->grads; r = 1; c = a->nparams; break;
        case GPT2_T_ADAM_M: off = a->adam_m; r = 1; c = a->nparams; break;
        case GPT2_T_ADAM_V: off = a->adam_v; r = 1; c = a->nparams; break;
        case GPT2_T_PARAMS_BF16:
            if (a->dtype != GPT2_BF16) return fail(GPT2_E_INVAL, "no bf16 copy in fp32 mode");
            off = a->params16; r = 1; c = a->nparams; dt = GPT2_BF16; break;
        case GPT2_T_ENCODED: off = a->encoded; r = BT; c = C; dt = act; break;
        case GPT2_T_LNF: off = a->lnf; r = BT; c = C; dt = act; break;
        case GPT2_T_LNF_STATS: off = a->lnfs; r = BT; c = 2; break;
        case GPT2_T_LOGITS: off = a->logits; r = BT; c = a->cfg.vocab_size; ld = a->Vp; dt = act; break;
        case GPT2_T_LOSSES: off = a->losses; r = BT; c = 1; break;
        case GPT2_T_LOSS: off = a->loss; r = 1; c = 1; break;
        case GPT2_T_LN1: off = x->ln1; r = BT; c = C; dt = act; break;
        case GPT2_T_LN1_STATS: off = x->ln1s; r = BT; c = 2; break;
        case GPT2_T_QKV: off = x->qkv; r = BT; c = 3 * C; dt = act; break;
        case GPT2_T_ATTY: off = x->atty; r = BT; c = C; dt = act; break;
        case GPT2_T_ATT_LSE: off = x->lse; r = (int64_t)a->B * NH; c = a->T; break;
        case GPT2_T_RESIDUAL2: off = x->res2; r = BT; c = C; dt = act; break;
        case GPT2_T_LN2: off = x->ln2; r = BT; c = C; dt = act; break;
        case GPT2_T_LN2_STATS: off = x->ln2s; r = BT; c = 2; break;
        case GPT2_T_FCH: off = x->fch; r = BT; c = a->F1; dt = act; break;
        case GPT2_T_FCH_GELU: off = x->fchg; r = BT; c = a->F2; dt = act; break;
        case GPT2_T_RESIDUAL3: off = x->res3; r = BT; c = C; dt = act; break;
        default: return fail(GPT2_E_INVAL, "unknown tensor id");
    }
    if (ld < 0) ld = c;
    if (byte_offset) *byte_offset = off;
    if (rows) *rows = r;
    if (cols) *cols = c;
    if (row_stride) *row_stride = ld;
    if (dtype) *dtype = dt;
    return GPT2_OK;
}

// ---------------------------------------------------------------- generation
int gpt2_gen_alloc(gpt2_arena* a, int32_t batch, int32_t max_len, void* device_base, size_t device_bytes,
                   size_t* required_bytes, gpt2_gen** out) {
    if (out) *out = nullptr;
    if (!a) return fail(GPT2_E_INVAL, "arena is NULL");
    if (a->dtype != GPT2_BF16) return fail(GPT2_E_INVAL, "generation needs a bf16 arena");
    if (a->block != GPT2_BLOCK_GPT2) return fail(GPT2_E_INVAL, "generation is built for the GPT-2 block");
    if (a->hs != 64) return fail(GPT2_E_INVAL, "generation needs head size 64");
    if (batch < 1 || batch > 16) return fail(GPT2_E_INVAL, "batch must be in 1..16");
    if (max_len < 1 || max_len > a->cfg.max_seq_len) return fail(GPT2_E_INVAL, "max_len must be in 1..max_seq_len");
    if (a->cfg.channels > 2048) return fail(GPT2_E_INVAL, "generation needs channels <= 2048");
    const size_t C = a->cfg.channels, L = a->cfg.num_layers, Bg = batch;
    gpt2_gen g{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t r = o;
        o = align_up(o + bytes);
        return r;
    };
    g.cache = take(L * Bg * max_len * 3 * C * 2);
    for (auto& r : g.res) r = take(Bg * C * 2);
    g.atty = take(Bg * C * 2);
    g.fchg = take(Bg * 4 * C * 2);
    g.lnf = take(Bg * C * 2);
    g.stats = take(Bg * 2 * 4);
    if (required_bytes) *required_bytes = o;
    if (!device_base) return GPT2_OK;
    if ((uintptr_t)device_base % kAlign) return fail(GPT2_E_ALIGN, "device_base must be 256-byte aligned");
    if (device_bytes < o) return fail(GPT2_E_SIZE, "device buffer too small: need " + std::to_string(o) + " bytes");
    if (!out) return fail(GPT2_E_INVAL, "out is NULL");
    gpt2_gen* h = new (std::nothrow) gpt2_gen(g);
    if (!h) return fail(GPT2_E_INVAL, "host allocation failed");
    h->a = a;
    h->batch = batch;
    h->max_len = max_len;
    h->len = 0;
    h->ready = false;
    h->base = (char*)device_base;
    *out = h;
    return GPT2_OK;
}

int gpt2_gen_free(gpt2_gen* g) {
    delete g;
    return GPT2_OK;
}

int gpt2_gen_length(const gpt2_gen* g) { return g ? g->len : -1; }

int gpt2_gen_prefill(gpt2_gen* g, const int32_t* d_tokens, int32_t n, float* d_logits, void* stream) {
    if (!g || !d_tokens || !d_logits) return fail(GPT2_E_INVAL, "generation state, tokens and logits are required");
    gpt2_arena* a = g->a;
    if (n < 1 || n > g->max_len) return fail(GPT2_E_SIZE, "prompt length must be in 1..max_len");
    if ((int64_t)g->batch * n > (int64_t)a->B * a->T)
        return fail(GPT2_E_SIZE, "batch * prompt length exceeds the arena's B * T rows");
    hipStream_t s = (hipStream_t)stream;
    g->ready = false;
    a->loss_ready = false;  // the arena's activations now describe the prompt
    a->inputs = nullptr;
    Model<bf16> m(a, s, g->batch, n);
    int rc = m.forward(d_tokens, nullptr);
    if (rc) return rc;
    const size_t C3 = 3 * (size_t)a->cfg.channels;
    for (int l = 0; l < a->cfg.num_layers; ++l) {
        char* dst = g->base + g->cache + (size_t)l * g->batch * g->max_len * C3 * 2;
        if (hipMemcpy2DAsync(dst, (size_t)g->max_len * C3 * 2, at<bf16>(a, a->la[l].qkv), (size_t)n * C3 * 2,
                             (size_t)n * C3 * 2, g->batch, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return fail(GPT2_E_HIP, "cache copy failed");
    }
    CHECK(logits_rows(d_logits, at<bf16>(a, a->logits), g->batch, a->cfg.vocab_size, a->Vp, n, n - 1, s), "logits");
    g->len = n;
    g->ready = true;
    return GPT2_OK;
}

int gpt2_gen_decode(gpt2_gen* g, const int32_t* d_tokens, float* d_logits, void* stream) {
    int rc = decode_check(g, d_tokens, d_logits);
    if (rc) return rc;
    const DecodeRows rows{g->base, {g->res[0], g->res[1], g->res[2]}, g->atty, g->fchg, g->lnf, g->stats};
    return decode_step(g, d_tokens, d_logits, (hipStream_t)stream, rows);
}

int gpt2_gen_decode_noalloc(gpt2_gen* g, const int32_t* d_tokens, float* d_logits, void* stream) {
    if (!g) return fail(GPT2_E_INVAL, "generation state is NULL");
    size_t need = 0;
    const DecodeRows lay = decode_rows_layout(g->batch, g->a->cfg.channels, nullptr, &need);
    if (need > kDecodeScratchBytes)
        return fail(GPT2_E_SIZE, "decode rows need " + std::to_string(need) + " bytes, more than the " +
                                     std::to_string(kDecodeScratchBytes) +
                                     "-byte static scratch (batch * channels at most about 19660)");
    int rc = decode_check(g, d_tokens, d_logits);
    if (rc) return rc;
    char* ptr = nullptr;
    if ((rc = decode_scratch_ptr(&ptr))) return rc;
    DecodeRows rows = lay;
    rows.base = ptr;
    return decode_step(g, d_tokens, d_logits, (hipStream_t)stream, rows);
}

// Host-side top-k sampling ("GPT-2 from scratch with torch", 生成样本): keep the k largest
// logits of a row (equal logits: the lower token id first), weight them by
// exp((z - z_max) / temperature), and take the first of them, in descending order,
// whose running sum of weights exceeds u * (sum of weights).
int gpt2_sample_topk(const float* logits, int32_t rows, int32_t V, int64_t ld, int32_t k, float temperature,
                     const float* uniforms, int32_t* tokens_out) {
    if (!logits || !uniforms || !tokens_out) return fail(GPT2_E_INVAL, "logits, uniforms and tokens_out are required");
    if (rows < 0 || V < 1 || ld < V) return fail(GPT2_E_INVAL, "bad logits shape");
    if (k < 1) return fail(GPT2_E_INVAL, "k must be >= 1");
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(GPT2_E_INVAL, "temperature must be > 0");
    const int kk = std::min(k, V);
    std::vector<int32_t> idx(V);
    for (int32_t r = 0; r < rows; ++r) {
        const float u = uniforms[r];
        if (!(u >= 0.f && u < 1.f)) return fail(GPT2_E_INVAL, "uniforms must lie in [0, 1)");
        const float* z = logits + (int64_t)r * ld;
        auto key = [&](int32_t i) { return std::isnan(z[i]) ? -INFINITY : z[i]; };  // NaN ranks last
        for (int32_t i = 0; i < V; ++i) idx[i] = i;
        std::partial_sort(idx.begin(), idx.begin() + kk, idx.end(), [&](int32_t x, int32_t y) {
            const float a = key(x), b = key(y);
            return a > b || (a == b && x < y);
        });
        const double zmax = key(idx[0]);
        if (!std::isfinite(zmax)) {  // an infinite logit leads, or nothing is finite: take the leader
            tokens_out[r] = idx[0];
            continue;
        }
        std::vector<double> w(kk);
        double total = 0.0;
        for (int i = 0; i < kk; ++i) {
            w[i] = std::exp(((double)key(idx[i]) - zmax) / (double)temperature);
            total += w[i];
        }
        const double target = (double)u * total;
        double run = 0.0;
        int32_t pick = idx[kk - 1];
        for (int i = 0; i < kk; ++i) {
            run += w[i];
            if (run > target) {
                pick = idx[i];
                break;
            }
        }
        tokens_out[r] = pick;
    }
    return GPT2_OK;
}

}  // extern "C"
