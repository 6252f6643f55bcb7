// Host-side file I/O of the library: token streams, parameter-order permutations and
// checkpoints (no device code; the caller moves the arrays to and from the arena).
//
// Token streams follow the llm.c page ("1000 行 C 代码完成 GPT-2 训练的 LLM.c", 快速开始吧):
// a .bin file is a raw stream of int32 token ids.  A batch of B sequences of T tokens
// takes B*T + 1 consecutive ids, inputs the first B*T and targets the same shifted by
// one, and batch i starts at id i*B*T.  The run banner on that page counts n / (B*T)
// batches (32768 ids -> 128, 305260 -> 1192 at B*T = 256), so when n is a multiple of
// B*T the last batch's final target would lie past the end: it wraps to id 0.  Weight files follow the 3000-byte C page ("GPT-2ベースの3000バイトCで実装さ
// れたChatGPTクローン", 重みの読み込み): one flat array of 32-bit floats in a fixed order,
// with the blocks of the layers stored in the lexicographic order of their decimal
// index (0, 1, 10, 11, 2, ...), which a permutation puts back into numeric order.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

namespace {

int io_fail(int code, const std::string& msg) { return gpt2::report_error(code, msg.c_str()); }

// Parameter counts of the pieces of the layer-major order: wte, wpe, L layer blocks, ln_f.
bool param_pieces(const gpt2_config* c, int64_t* head, int64_t* layer, int64_t* tail) {
    if (!c || c->channels <= 0 || c->num_layers <= 0 || c->vocab_size <= 0 || c->max_seq_len <= 0) return false;
    const int64_t C = c->channels;
    *head = ((int64_t)c->vocab_size + c->max_seq_len) * C;
    *layer = 12 * C * C + 13 * C;  // ln_1 2C, c_attn 3C^2+3C, attn c_proj C^2+C, ln_2 2C, c_fc 4C^2+4C, c_proj 4C^2+C
    *tail = 2 * C;
    return true;
}

// Storage slot of layer l in lexicographic order of the decimal indices 0 .. L-1.
std::vector<int> lexicographic_layers(int L) {
    std::vector<int> ids(L);
    for (int i = 0; i < L; ++i) ids[i] = i;
    std::sort(ids.begin(), ids.end(), [](int a, int b) { return std::to_string(a) < std::to_string(b); });
    return ids;  // ids[k] = the layer stored k-th
}

constexpr int32_t kMagic = 0x32545047;  // "GPT2" little endian
constexpr int32_t kVersion = 1;

}  // namespace

extern "C" {

int64_t gpt2_tokens_count(const char* path) {
    if (!path) return io_fail(GPT2_E_INVAL, "path is NULL");
    FILE* f = fopen(path, "rb");
    if (!f) return io_fail(GPT2_E_INVAL, std::string("cannot open ") + path);
    fseek(f, 0, SEEK_END);
    const long bytes = ftell(f);
    fclose(f);
    if (bytes < 0 || bytes % 4) return io_fail(GPT2_E_SIZE, "token file size is not a multiple of 4 bytes");
    return bytes / 4;
}

int gpt2_tokens_batch(const char* path, int32_t B, int32_t T, int64_t batch, int32_t* inputs, int32_t* targets) {
    if (!path || !inputs || !targets) return io_fail(GPT2_E_INVAL, "path, inputs and targets are required");
    if (B < 1 || T < 1) return io_fail(GPT2_E_INVAL, "need B, T >= 1");
    const int64_t n = gpt2_tokens_count(path);
    if (n < 0) return (int)n;
    const int64_t bt = (int64_t)B * T, nb = n / bt;
    if (batch < 0 || batch >= nb) return io_fail(GPT2_E_SIZE, "batch index outside 0 .. num_batches - 1");
    std::vector<int32_t> buf(bt + 1);
    FILE* f = fopen(path, "rb");
    if (!f) return io_fail(GPT2_E_INVAL, std::string("cannot open ") + path);
    const int64_t start = batch * bt, avail = std::min(bt + 1, n - start);  // avail is bt or bt + 1
    bool ok = fseek(f, (long)(start * 4), SEEK_SET) == 0 && fread(buf.data(), 4, avail, f) == (size_t)avail;
    if (ok && avail == bt) ok = fseek(f, 0, SEEK_SET) == 0 && fread(buf.data() + bt, 4, 1, f) == 1;  // wrap
    fclose(f);
    if (!ok) return io_fail(GPT2_E_SIZE, "short read");
    memcpy(inputs, buf.data(), bt * 4);
    memcpy(targets, buf.data() + 1, bt * 4);
    return GPT2_OK;
}

int gpt2_params_permute(const gpt2_config* cfg, const float* src, float* dst, int32_t from_order, int32_t to_order) {
    int64_t head, layer, tail;
    if (!param_pieces(cfg, &head, &layer, &tail)) return io_fail(GPT2_E_INVAL, "bad config");
    if (!src || !dst || src == dst) return io_fail(GPT2_E_INVAL, "src and dst must be distinct arrays");
    auto valid = [](int32_t o) { return o == GPT2_ORDER_NUMERIC || o == GPT2_ORDER_LEXICOGRAPHIC; };
    if (!valid(from_order) || !valid(to_order)) return io_fail(GPT2_E_INVAL, "unknown layer order");
    const int L = cfg->num_layers;
    const std::vector<int> lex = lexicographic_layers(L);
    // slot of layer l in each order
    auto slot = [&](int32_t order, int l) {
        if (order == GPT2_ORDER_NUMERIC) return l;
        return (int)(std::find(lex.begin(), lex.end(), l) - lex.begin());
    };
    memcpy(dst, src, head * sizeof(float));
    for (int l = 0; l < L; ++l)
        memcpy(dst + head + (int64_t)slot(to_order, l) * layer, src + head + (int64_t)slot(from_order, l) * layer,
               layer * sizeof(float));
    memcpy(dst + head + (int64_t)L * layer, src + head + (int64_t)L * layer, tail * sizeof(float));
    return GPT2_OK;
}

int gpt2_checkpoint_write(const char* path, const gpt2_config* cfg, int32_t step, const float* params, const float* m,
                          const float* v) {
    int64_t head, layer, tail;
    if (!path || !params || !param_pieces(cfg, &head, &layer, &tail)) return io_fail(GPT2_E_INVAL, "bad arguments");
    if ((m == nullptr) != (v == nullptr)) return io_fail(GPT2_E_INVAL, "give both AdamW moments or neither");
    const int64_t n = head + (int64_t)cfg->num_layers * layer + tail;
    const int32_t hdr[16] = {kMagic, kVersion, cfg->max_seq_len, cfg->vocab_size, cfg->num_layers, cfg->num_heads,
                             cfg->channels, m ? 1 : 0, step, 0, 0, 0, 0, 0, 0, 0};
    const std::string tmp = std::string(path) + ".tmp";
    FILE* f = fopen(tmp.c_str(), "wb");
    if (!f) return io_fail(GPT2_E_INVAL, "cannot create " + tmp);
    bool ok = fwrite(hdr, 4, 16, f) == 16 && fwrite(params, 4, n, f) == (size_t)n;
    if (ok && m) ok = fwrite(m, 4, n, f) == (size_t)n && fwrite(v, 4, n, f) == (size_t)n;
    ok = (fclose(f) == 0) && ok;
    if (!ok || rename(tmp.c_str(), path) != 0) {
        remove(tmp.c_str());
        return io_fail(GPT2_E_SIZE, std::string("write failed: ") + path);
    }
    return GPT2_OK;
}

int gpt2_checkpoint_read(const char* path, const gpt2_config* cfg, int32_t* step, float* params, float* m, float* v,
                         int32_t* has_moments) {
    int64_t head, layer, tail;
    if (!path || !params || !param_pieces(cfg, &head, &layer, &tail)) return io_fail(GPT2_E_INVAL, "bad arguments");
    const int64_t n = head + (int64_t)cfg->num_layers * layer + tail;
    FILE* f = fopen(path, "rb");
    if (!f) return io_fail(GPT2_E_INVAL, std::string("cannot open ") + path);
    int32_t hdr[16];
    bool ok = fread(hdr, 4, 16, f) == 16;
    if (ok && (hdr[0] != kMagic || hdr[1] != kVersion)) {
        fclose(f);
        return io_fail(GPT2_E_INVAL, "not a checkpoint of this library (magic / version)");
    }
    if (ok && (hdr[2] != cfg->max_seq_len || hdr[3] != cfg->vocab_size || hdr[4] != cfg->num_layers ||
               hdr[5] != cfg->num_heads || hdr[6] != cfg->channels)) {
        fclose(f);
        return io_fail(GPT2_E_INVAL, "checkpoint model shape differs from cfg");
    }
    ok = ok && fread(params, 4, n, f) == (size_t)n;
    const bool moments = ok && hdr[7] == 1;
    if (moments && m && v) ok = fread(m, 4, n, f) == (size_t)n && fread(v, 4, n, f) == (size_t)n;
    fclose(f);
    if (!ok) return io_fail(GPT2_E_SIZE, "short read");
    if (step) *step = hdr[8];
    if (has_moments) *has_moments = moments ? 1 : 0;
    return GPT2_OK;
}

}  // extern "C"
