// runtime.hip — host side of the library: the C ABI of include/decfwd.h.
//
// Load follows page "Execution contract", section "Load phase": validate
// the config and the tensor table, upload the weights, precompute the RoPE
// cos/sin cache. Memory follows section "Memory lifecycle": weights live as
// long as the model; one KV cache sized to max context, appended on every
// step and cleared by reset; activations come from a frame allocator with
// exact-size buckets that is reset at the start of every forward. Errors are
// structured codes with a message naming the tensor / field / bytes (section
// "Error semantics"); a failed call never aborts and never falls back.
#include "kernels.h"

#include "../../include/decfwd.h"

static_assert(dfk::MAX_WIDTH == DF_MAX_WIDTH, "kernel width limit matches the header");
static_assert(dfk::GEMM_PLAN_128x128 == DF_GEMM_T128x128 && dfk::GEMM_PLAN_128x256 == DF_GEMM_T128x256 &&
                  dfk::GEMM_PLAN_256x256 == DF_GEMM_T256x256 &&
                  dfk::GEMM_PLAN_256x256_LDS == DF_GEMM_T256x256_LDS &&
                  dfk::GEMM_PLAN_256x192_LDS == DF_GEMM_T256x192_LDS &&
                  dfk::GEMM_PLAN_TILE_MASK == DF_GEMM_TILE_MASK &&
                  dfk::GEMM_PLAN_Q8_IN_GEMM == DF_GEMM_Q8_IN_GEMM &&
                  dfk::GEMM_PLAN_DEQUANT_FIRST == DF_GEMM_Q8_DEQUANT_FIRST &&
                  dfk::GEMM_PLAN_SPLIT_SHIFT == DF_GEMM_SPLIT_SHIFT && dfk::GEMM_PLAN_SPLIT_MASK == DF_GEMM_SPLIT_MASK,
              "GEMM plan codes match the header");

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

using namespace dfk;

namespace dfk {
LaunchTiming& launch_timing()
{
    thread_local LaunchTiming t;
    return t;
}
}  // namespace dfk

namespace {

thread_local std::string g_load_error;

std::string fmt(const char* f, ...)
{
    char buf[1024];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    return buf;
}

struct Fail {
    df_status code;
    std::string msg;
};

// ---------------------------------------------------------------------------
// Frame allocator (page "Execution contract", "Memory lifecycle",
// "Activations"): buffers bucketed by (exact byte size, usage); reset()
// makes every buffer of the previous forward available again. Within a
// bucket buffers are handed out in a fixed order from a cursor, so a forward
// that makes the same requests gets the same addresses every time.
// ---------------------------------------------------------------------------
enum Usage { USAGE_DEVICE = 0 };

class FramePool {
public:
    void* alloc(size_t bytes, int usage, Fail* err)
    {
        auto key = std::make_pair(bytes, usage);
        auto& bucket = pool_[key];
        size_t& cur = cursor_[key];
        if (cur == bucket.size()) {
            void* p = nullptr;
            if (hipMalloc(&p, bytes ? bytes : 1) != hipSuccess) {
                (void)hipGetLastError();
                *err = {DF_ERR_OUT_OF_MEMORY,
                        fmt("frame allocator: hipMalloc of %zu bytes failed", bytes)};
                return nullptr;
            }
            bucket.push_back(p);
            total_ += bytes;
        }
        return bucket[cur++];
    }
    void reset()
    {
        for (auto& kv : cursor_) kv.second = 0;
    }
    void release()
    {
        for (auto& kv : pool_)
            for (void* p : kv.second) (void)hipFree(p);
        pool_.clear();
        cursor_.clear();
        total_ = 0;
    }
    size_t bytes() const { return total_; }

private:
    std::map<std::pair<size_t, int>, std::vector<void*>> pool_;
    std::map<std::pair<size_t, int>, size_t> cursor_;
    size_t total_ = 0;
};

// Device memory of the weights, the position caches and the zero block:
// shared by a model and every session opened on it, freed when the last of
// them is freed.
struct WeightStore {
    int device = 0;
    std::vector<void*> allocs;
    ~WeightStore()
    {
        if (allocs.empty()) return;
        (void)hipSetDevice(device);
        for (void* p : allocs) (void)hipFree(p);
    }
};

struct Layer {
    Weight wqkv, wo, wgu, wd;  // [q;k;v], o, [gate;up], down
    float* attn_norm = nullptr;
    float* ffn_norm = nullptr;
    float* q_norm = nullptr;
    float* k_norm = nullptr;
    float* bqkv = nullptr;     // qwen2: [q bias | k bias | v bias]
    float* post_attn_norm = nullptr;  // gemma3: rms_norm of o before the add
    float* post_ffn_norm = nullptr;   // gemma3: rms_norm of down before the add
    bool local = false;        // attends through the sliding window, local rope theta
};

}  // namespace

// ---------------------------------------------------------------------------
// Fixed staging for df_forward_noalloc: the decode step's activations (x,
// q|k|v, attention output, gated FFN activation, gemma3's norm input) in one
// file-scope device array, so that the call allocates nothing. Each GPU the
// library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, not device memory: host code uses
// only the per-device address hipGetSymbolAddress gives (noalloc_scratch).
// ---------------------------------------------------------------------------
constexpr size_t NOALLOC_SCRATCH_BYTES = DF_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;  // device ordinal -> address of its `scratch`

// Once per device, with that device current: the device address of the
// array. Called by df_load.
bool noalloc_scratch_init(int dev, std::string* err)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_addr.count(dev)) return true;
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !p) {
        (void)hipGetLastError();
        *err = fmt("backend init: hipGetSymbolAddress of the fixed staging array failed on device %d (%s)",
                   dev, hipGetErrorString(r));
        return false;
    }
    g_scratch_addr[dev] = p;
    return true;
}

void* noalloc_scratch(int dev)
{
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    return it == g_scratch_addr.end() ? nullptr : it->second;
}
}  // namespace

struct df_model {
    df_config cfg{};
    int device = 0;
    hipStream_t stream = nullptr;
    bool own_stream = false;
    std::string err;
    std::atomic<int> busy{0};
    int32_t kv_len = 0;

    std::vector<void*> allocs;  // this conversation's device allocations
    std::shared_ptr<WeightStore> wstore;  // weights, shared with sessions
    std::vector<void*>* alloc_to = nullptr;  // where dev_alloc records (null: allocs)
    int64_t weight_bytes = 0, kv_bytes = 0;
    int32_t rope_rows = 0;  // positions the cos/sin table covers

    Weight embd, out;
    float* out_norm = nullptr;
    std::vector<Layer> layers;
    float* kc = nullptr;  // [L][n_kv][max_ctx][hd]
    float* vc = nullptr;
    // f16 copies for the bulk-prefill attention (null where it reads kc / vc):
    // K [L][n_kv][max_ctx][hd], V transposed [L][n_kv][hd][max_ctx]
    uint16_t* k16 = nullptr;
    int* gemm_tickets = nullptr;  // GEMM_SPLIT_TICKETS counters, zero between GEMMs (split tiles)
    uint16_t* vt16 = nullptr;
    float* cos_t = nullptr;  // [max_ctx][hd/2]
    float* sin_t = nullptr;
    float* cos_l = nullptr;  // local layers' table (rope_theta_local), else cos_t
    float* sin_l = nullptr;
    DevState* state = nullptr;
    float* attn_part = nullptr;
    int* argmax_out = nullptr;
    uint16_t* zeros = nullptr;  // 256 zero bytes: source of out-of-range GEMM chunks
    int* gen_tokens = nullptr;  // [max_ctx]

    FramePool pool;

    // Captured decode step (+ argmax) for df_generate, replayed once per
    // token; valid while its buffers are the ones the pool hands out.
    hipGraphExec_t gen_exec = nullptr;
    std::vector<void*> gen_key;

    // df_profile: event pairs around the launches of one kernel class.
    int prof_kernel = -1;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_events;
    size_t prof_used = 0;
    int64_t prof_launches = 0;
    double prof_ms = 0;

    double load_ms = 0;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    int ev_kind = 0;  // 0 none, 1 step, 2 prefill
    double last_prefill_ms = 0, last_step_ms = 0;
    int64_t n_forward = 0;
};

namespace {

void* dev_alloc(df_model* m, size_t bytes, const char* what, Fail* err)
{
    void* p = nullptr;
    if (hipMalloc(&p, bytes ? bytes : 1) != hipSuccess) {
        (void)hipGetLastError();
        *err = {DF_ERR_OUT_OF_MEMORY,
                fmt("hipMalloc of %zu bytes for %s failed", bytes, what)};
        return nullptr;
    }
    (m->alloc_to ? *m->alloc_to : m->allocs).push_back(p);
    return p;
}

void release(df_model* m)
{
    if (!m) return;
    if (m->stream) (void)hipStreamSynchronize(m->stream);
    for (void* p : m->allocs) (void)hipFree(p);
    m->allocs.clear();
    for (auto& ev : m->prof_events) {
        (void)hipEventDestroy(ev.first);
        (void)hipEventDestroy(ev.second);
    }
    m->prof_events.clear();
    if (m->gen_exec) (void)hipGraphExecDestroy(m->gen_exec);
    m->gen_exec = nullptr;
    m->pool.release();
    if (m->ev0) (void)hipEventDestroy(m->ev0);
    if (m->ev1) (void)hipEventDestroy(m->ev1);
    if (m->own_stream && m->stream) (void)hipStreamDestroy(m->stream);
    m->stream = nullptr;
    m->wstore.reset();
}

// ---------------------------------------------------------------------------
// Validation (page "Execution contract", "Load phase", step 3: config schema
// and tensor completeness). Host only: runs before any HIP call.
// ---------------------------------------------------------------------------
bool cfg_fail(Fail* e, const char* field, const std::string& reason)
{
    *e = {DF_ERR_INVALID_CONFIG, fmt("invalid config: %s %s", field, reason.c_str())};
    return false;
}

bool validate_config(const df_config* c, Fail* e)
{
    if (!c) { *e = {DF_ERR_INVALID_ARGUMENT, "config is NULL"}; return false; }
    if (c->arch != DF_ARCH_LLAMA && c->arch != DF_ARCH_QWEN3 && c->arch != DF_ARCH_QWEN2 &&
        c->arch != DF_ARCH_GEMMA3)
        return cfg_fail(e, "arch", fmt("= %d: expected 0 (llama), 1 (qwen3), 2 (qwen2) or 3 (gemma3)",
                                       c->arch));
    if (c->sliding_window < 0)
        return cfg_fail(e, "sliding_window", fmt("= %d: expected >= 0", c->sliding_window));
    if (c->sliding_window > 0 && c->window_pattern < 1)
        return cfg_fail(e, "window_pattern", fmt("= %d: expected >= 1 with a sliding window",
                                                 c->window_pattern));
    if (!(c->rope_theta_local >= 0) || !std::isfinite(c->rope_theta_local))
        return cfg_fail(e, "rope_theta_local", fmt("= %g: expected a finite value >= 0 (0: rope_theta)",
                                                   c->rope_theta_local));
    if (c->rope_pairing != DF_ROPE_HALVES && c->rope_pairing != DF_ROPE_ADJACENT)
        return cfg_fail(e, "rope_pairing", fmt("= %d: expected 0 (halves) or 1 (adjacent)",
                                               c->rope_pairing));
    if (c->n_layers < 0 || c->n_layers > 4096)
        return cfg_fail(e, "n_layers", fmt("= %d: expected 0..4096", c->n_layers));
    if (c->d_model <= 0 || c->d_model % 32 || c->d_model > DF_MAX_WIDTH)
        return cfg_fail(e, "d_model", fmt("= %d: expected a multiple of 32 in 32..%d", c->d_model,
                                          DF_MAX_WIDTH));
    if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128 &&
        c->head_dim != 256)
        return cfg_fail(e, "head_dim", fmt("= %d: expected 16, 32, 64, 128 or 256", c->head_dim));
    if (c->n_kv_heads <= 0 || c->n_heads <= 0 || c->n_heads % c->n_kv_heads)
        return cfg_fail(e, "n_heads", fmt("= %d with n_kv_heads = %d: n_kv_heads must divide n_heads",
                                          c->n_heads, c->n_kv_heads));
    {
        const int G = c->n_heads / c->n_kv_heads;
        if (G > ATTN_MAX_GROUP)
            return cfg_fail(e, "n_heads", fmt("/ n_kv_heads = %d: expected at most %d query heads "
                                              "per KV head", G, ATTN_MAX_GROUP));
    }
    if (int64_t(c->n_heads) * c->head_dim > DF_MAX_WIDTH || (c->n_heads * c->head_dim) % 32)
        return cfg_fail(e, "n_heads", fmt("* head_dim = %lld: expected a multiple of 32 up to %d",
                                          (long long)c->n_heads * c->head_dim, DF_MAX_WIDTH));
    if (c->ffn_dim <= 0 || c->ffn_dim % 32 || c->ffn_dim > DF_MAX_WIDTH)
        return cfg_fail(e, "ffn_dim", fmt("= %d: expected a multiple of 32 in 32..%d", c->ffn_dim,
                                          DF_MAX_WIDTH));
    if (c->vocab <= 0)
        return cfg_fail(e, "vocab", fmt("= %d: expected >= 1", c->vocab));
    if (c->max_ctx <= 0 || c->max_ctx > (1 << 20))
        return cfg_fail(e, "max_ctx", fmt("= %d: expected 1..1048576", c->max_ctx));
    if (!(c->rope_theta > 0) || !std::isfinite(c->rope_theta))
        return cfg_fail(e, "rope_theta", fmt("= %g: expected a finite value > 0", c->rope_theta));
    if (!(c->rms_eps >= 0) || !std::isfinite(c->rms_eps))
        return cfg_fail(e, "rms_eps", fmt("= %g: expected a finite value >= 0", c->rms_eps));
    return true;
}

const char* dtype_name(int d)
{
    return d == DF_F32 ? "f32" : d == DF_F16 ? "f16" : d == DF_Q8_32 ? "q8_32" : "unknown";
}

uint64_t expected_bytes(int dtype, int64_t rows, int64_t cols)
{
    if (dtype == DF_F32) return uint64_t(rows * cols) * 4;
    if (dtype == DF_F16) return uint64_t(rows * cols) * 2;
    return uint64_t(rows) * uint64_t(cols / 32) * 34;
}

enum Kind { K_EMBED, K_NORM, K_MATMUL, K_BIAS };

// gemma3's embedding scale (the "scale" step after embed): f32(sqrt(d_model)).
float embed_scale(const df_config& c)
{
    return c.arch == DF_ARCH_GEMMA3 ? float(std::sqrt(double(c.d_model))) : 1.0f;
}

const char* arch_name(int a)
{
    return a == DF_ARCH_QWEN3 ? "qwen3" : a == DF_ARCH_QWEN2 ? "qwen2"
         : a == DF_ARCH_GEMMA3 ? "gemma3" : "llama";
}

struct Need {
    std::string name;
    Kind kind;
    int64_t rows, cols;
    bool required;
    std::string required_by;
};

std::vector<Need> required_tensors(const df_config* c)
{
    const int64_t d = c->d_model, hd = c->head_dim, F = c->ffn_dim, V = c->vocab;
    const int64_t qd = int64_t(c->n_heads) * hd, kvd = int64_t(c->n_kv_heads) * hd;
    std::vector<Need> v;
    v.push_back({"token_embd.weight", K_EMBED, V, d, true, "embed"});
    for (int i = 0; i < c->n_layers; ++i) {
        const std::string b = "blk." + std::to_string(i) + ".";
        const std::string L = "layer " + std::to_string(i);
        v.push_back({b + "attn_norm.weight", K_NORM, 1, d, true, L + " rms_norm (attention)"});
        v.push_back({b + "attn_q.weight", K_MATMUL, qd, d, true, L + " q matmul"});
        v.push_back({b + "attn_k.weight", K_MATMUL, kvd, d, true, L + " k matmul"});
        v.push_back({b + "attn_v.weight", K_MATMUL, kvd, d, true, L + " v matmul"});
        if (c->arch == DF_ARCH_QWEN2) {
            v.push_back({b + "attn_q.bias", K_BIAS, 1, qd, true, L + " add_bias q"});
            v.push_back({b + "attn_k.bias", K_BIAS, 1, kvd, true, L + " add_bias k"});
            v.push_back({b + "attn_v.bias", K_BIAS, 1, kvd, true, L + " add_bias v"});
        }
        if (c->arch == DF_ARCH_QWEN3 || c->arch == DF_ARCH_GEMMA3) {
            v.push_back({b + "attn_q_norm.weight", K_NORM, 1, hd, true, L + " norm_heads q"});
            v.push_back({b + "attn_k_norm.weight", K_NORM, 1, hd, true, L + " norm_heads k"});
        }
        if (c->arch == DF_ARCH_GEMMA3) {
            v.push_back({b + "post_attention_norm.weight", K_NORM, 1, d, true, L + " rms_norm of o"});
            v.push_back({b + "post_ffw_norm.weight", K_NORM, 1, d, true, L + " rms_norm of down"});
        }
        v.push_back({b + "attn_output.weight", K_MATMUL, d, qd, true, L + " o matmul"});
        v.push_back({b + "ffn_norm.weight", K_NORM, 1, d, true, L + " rms_norm (ffn)"});
        v.push_back({b + "ffn_gate.weight", K_MATMUL, F, d, true, L + " gate matmul"});
        v.push_back({b + "ffn_up.weight", K_MATMUL, F, d, true, L + " up matmul"});
        v.push_back({b + "ffn_down.weight", K_MATMUL, d, F, true, L + " down matmul"});
    }
    v.push_back({"output_norm.weight", K_NORM, 1, d, true, "final rms_norm"});
    v.push_back({"output.weight", K_MATMUL, V, d, false, "logits matmul"});
    return v;
}

bool validate_tensors(const df_config* c, const df_tensor* t, size_t n,
                      std::map<std::string, const df_tensor*>* found, Fail* e)
{
    if (n && !t) { *e = {DF_ERR_INVALID_ARGUMENT, "tensor table is NULL"}; return false; }
    const auto need = required_tensors(c);
    std::map<std::string, const Need*> by_name;
    for (const auto& nd : need) by_name[nd.name] = &nd;
    for (size_t i = 0; i < n; ++i) {
        if (!t[i].name) {
            *e = {DF_ERR_INVALID_ARGUMENT, fmt("tensor %zu has no name", i)};
            return false;
        }
        const std::string name = t[i].name;
        auto it = by_name.find(name);
        if (it == by_name.end()) {
            *e = {DF_ERR_INVALID_ARGUMENT,
                  fmt("tensor '%s' is not part of the %s step list with %d layers", name.c_str(),
                      arch_name(c->arch), c->n_layers)};
            return false;
        }
        if (found->count(name)) {
            *e = {DF_ERR_INVALID_ARGUMENT, fmt("tensor '%s' given twice", name.c_str())};
            return false;
        }
        const Need& nd = *it->second;
        const df_tensor& x = t[i];
        if (x.dtype != DF_F32 && x.dtype != DF_F16 && x.dtype != DF_Q8_32) {
            *e = {DF_ERR_UNSUPPORTED_OP, fmt("tensor '%s': dtype code %d is not f32, f16 or q8_32",
                                             name.c_str(), x.dtype)};
            return false;
        }
        if (nd.kind != K_MATMUL && x.dtype == DF_Q8_32) {
            *e = {DF_ERR_UNSUPPORTED_OP,
                  fmt("tensor '%s' (%s): q8_32 is supported for matmul weights only; "
                      "embeddings, norm weights and biases are f32 or f16",
                      name.c_str(), nd.required_by.c_str())};
            return false;
        }
        if (x.rows != nd.rows || x.cols != nd.cols) {
            *e = {DF_ERR_SHAPE_MISMATCH,
                  fmt("tensor '%s' (%s): expected shape [%lld, %lld], got [%lld, %lld]",
                      name.c_str(), nd.required_by.c_str(), (long long)nd.rows,
                      (long long)nd.cols, (long long)x.rows, (long long)x.cols)};
            return false;
        }
        if (x.dtype == DF_Q8_32 && x.cols % 32) {
            *e = {DF_ERR_SHAPE_MISMATCH, fmt("tensor '%s': q8_32 needs cols divisible by 32, got %lld",
                                             name.c_str(), (long long)x.cols)};
            return false;
        }
        const uint64_t want = expected_bytes(x.dtype, x.rows, x.cols);
        if (x.nbytes != want) {
            *e = {DF_ERR_WEIGHT_FORMAT_MISMATCH,
                  fmt("tensor '%s': declared %s [%lld, %lld] needs %llu bytes, got %llu",
                      name.c_str(), dtype_name(x.dtype), (long long)x.rows, (long long)x.cols,
                      (unsigned long long)want, (unsigned long long)x.nbytes)};
            return false;
        }
        if (!x.data) {
            *e = {DF_ERR_INVALID_ARGUMENT, fmt("tensor '%s': data is NULL", name.c_str())};
            return false;
        }
        (*found)[name] = &x;
    }
    for (const auto& nd : need) {
        if (nd.required && !found->count(nd.name)) {
            *e = {DF_ERR_MISSING_TENSOR, fmt("missing tensor '%s', required by %s",
                                             nd.name.c_str(), nd.required_by.c_str())};
            return false;
        }
    }
    // Fused launches need matching dtypes: q/k/v, gate/up, and one dtype for
    // every block matmul so that all layers run the same kernels.
    int block_dtype = -1;
    for (const auto& nd : need) {
        if (nd.kind != K_MATMUL || nd.name == "output.weight") continue;
        const int dt = (*found)[nd.name]->dtype;
        if (block_dtype < 0) block_dtype = dt;
        if (dt != block_dtype) {
            *e = {DF_ERR_WEIGHT_FORMAT_MISMATCH,
                  fmt("tensor '%s' is %s but the other block matmul weights are %s; "
                      "one dtype is required for all of them",
                      nd.name.c_str(), dtype_name(dt), dtype_name(block_dtype))};
            return false;
        }
    }
    return true;
}

// ---------------------------------------------------------------------------
// Upload.
// ---------------------------------------------------------------------------
bool check(hipError_t r, const char* what, Fail* e, df_status code = DF_ERR_BACKEND_INIT)
{
    if (r == hipSuccess) return true;
    (void)hipGetLastError();
    *e = {code, fmt("%s: %s", what, hipGetErrorString(r))};
    return false;
}

hipMemcpyKind kind_of(const df_tensor* t)
{
    return t->on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
}

// Concatenate matmul weights along rows into one device matrix.
bool upload_matrix(df_model* m, const std::vector<const df_tensor*>& parts,
                   Weight* w, const char* what, Fail* e)
{
    const int dt = parts[0]->dtype;
    const int64_t cols = parts[0]->cols;
    int64_t rows = 0;
    for (auto* p : parts) rows += p->rows;
    w->rows = rows;
    w->cols = cols;
    if (dt == DF_F32 || dt == DF_F16) {
        const size_t es = dt == DF_F32 ? 4 : 2;
        char* dst = static_cast<char*>(dev_alloc(m, size_t(rows * cols) * es, what, e));
        if (!dst) return false;
        size_t off = 0;
        for (auto* p : parts) {
            if (!check(hipMemcpyAsync(dst + off, p->data, p->nbytes, kind_of(p), m->stream),
                       what, e))
                return false;
            off += p->nbytes;
        }
        w->dtype = dt == DF_F32 ? W_F32 : W_F16;
        w->data = dst;
        w->scales = nullptr;
        m->weight_bytes += int64_t(rows * cols * es);
        return true;
    }
    // 8-bit blocks: value plane [rows][cols] and scale plane [rows][cols/32].
    int8_t* vals = static_cast<int8_t*>(dev_alloc(m, size_t(rows * cols), what, e));
    if (!vals) return false;
    uint16_t* sc = static_cast<uint16_t*>(dev_alloc(m, size_t(rows * (cols / 32)) * 2, what, e));
    if (!sc) return false;
    int64_t row0 = 0;
    for (auto* p : parts) {
        const uint8_t* src = static_cast<const uint8_t*>(p->data);
        void* staging = nullptr;
        if (!p->on_device) {
            if (!check(hipMalloc(&staging, p->nbytes), "staging for 8-bit repack", e,
                       DF_ERR_OUT_OF_MEMORY))
                return false;
            if (!check(hipMemcpyAsync(staging, p->data, p->nbytes, hipMemcpyHostToDevice,
                                      m->stream), what, e)) {
                (void)hipFree(staging);
                return false;
            }
            src = static_cast<const uint8_t*>(staging);
        }
        hipError_t r = launch_q8_split(src, p->rows, cols, vals + row0 * cols,
                                       sc + row0 * (cols / 32), m->stream);
        if (staging) {
            (void)hipStreamSynchronize(m->stream);
            (void)hipFree(staging);
        }
        if (!check(r, "8-bit repack", e)) return false;
        row0 += p->rows;
    }
    w->dtype = W_Q8;
    w->data = vals;
    w->scales = sc;
    m->weight_bytes += int64_t(rows * cols + rows * (cols / 32) * 2);
    return true;
}

// Convert one f32/f16 vector into f32 device memory at dst.
bool upload_vector_into(df_model* m, const df_tensor* t, float* dst, Fail* e)
{
    const int64_t n = t->rows * t->cols;
    const void* src = t->data;
    void* staging = nullptr;
    if (!t->on_device) {
        if (!check(hipMalloc(&staging, t->nbytes), "staging", e, DF_ERR_OUT_OF_MEMORY)) return false;
        if (!check(hipMemcpyAsync(staging, t->data, t->nbytes, hipMemcpyHostToDevice, m->stream),
                   t->name, e)) {
            (void)hipFree(staging);
            return false;
        }
        src = staging;
    }
    hipError_t r = launch_to_f32(src, t->dtype == DF_F32 ? W_F32 : W_F16, n, dst, m->stream);
    if (staging) {
        (void)hipStreamSynchronize(m->stream);
        (void)hipFree(staging);
    }
    if (!check(r, t->name, e)) return false;
    m->weight_bytes += n * 4;
    return true;
}

// Concatenate vectors into one f32 device vector.
bool upload_vectors(df_model* m, const std::vector<const df_tensor*>& parts, float** out,
                    const char* what, Fail* e)
{
    int64_t n = 0;
    for (auto* t : parts) n += t->rows * t->cols;
    float* dst = static_cast<float*>(dev_alloc(m, size_t(n) * 4, what, e));
    if (!dst) return false;
    int64_t off = 0;
    for (auto* t : parts) {
        if (!upload_vector_into(m, t, dst + off, e)) return false;
        off += t->rows * t->cols;
    }
    *out = dst;
    return true;
}

bool upload_norm(df_model* m, const df_tensor* t, float** out, Fail* e)
{
    return upload_vectors(m, {t}, out, t->name, e);
}

bool upload_embedding(df_model* m, const df_tensor* t, Weight* w, Fail* e)
{
    std::vector<const df_tensor*> parts{t};
    return upload_matrix(m, parts, w, t->name, e);
}

bool build_weights(df_model* m, const std::map<std::string, const df_tensor*>& T, Fail* e)
{
    const df_config& c = m->cfg;
    auto get = [&](const std::string& n) { return T.at(n); };
    if (!upload_embedding(m, get("token_embd.weight"), &m->embd, e)) return false;
    m->layers.resize(size_t(c.n_layers));
    for (int i = 0; i < c.n_layers; ++i) {
        const std::string b = "blk." + std::to_string(i) + ".";
        Layer& L = m->layers[size_t(i)];
        if (!upload_norm(m, get(b + "attn_norm.weight"), &L.attn_norm, e)) return false;
        if (!upload_matrix(m, {get(b + "attn_q.weight"), get(b + "attn_k.weight"),
                               get(b + "attn_v.weight")}, &L.wqkv, "q/k/v weights", e))
            return false;
        if (c.arch == DF_ARCH_QWEN2 &&
            !upload_vectors(m, {get(b + "attn_q.bias"), get(b + "attn_k.bias"),
                                get(b + "attn_v.bias")}, &L.bqkv, "q/k/v biases", e))
            return false;
        if (c.arch == DF_ARCH_QWEN3 || c.arch == DF_ARCH_GEMMA3) {
            if (!upload_norm(m, get(b + "attn_q_norm.weight"), &L.q_norm, e)) return false;
            if (!upload_norm(m, get(b + "attn_k_norm.weight"), &L.k_norm, e)) return false;
        }
        if (c.arch == DF_ARCH_GEMMA3) {
            if (!upload_norm(m, get(b + "post_attention_norm.weight"), &L.post_attn_norm, e)) return false;
            if (!upload_norm(m, get(b + "post_ffw_norm.weight"), &L.post_ffn_norm, e)) return false;
        }
        L.local = c.sliding_window > 0 && (i + 1) % c.window_pattern != 0;
        if (!upload_matrix(m, {get(b + "attn_output.weight")}, &L.wo, "o weight", e)) return false;
        if (!upload_norm(m, get(b + "ffn_norm.weight"), &L.ffn_norm, e)) return false;
        if (!upload_matrix(m, {get(b + "ffn_gate.weight"), get(b + "ffn_up.weight")}, &L.wgu,
                           "gate/up weights", e))
            return false;
        if (!upload_matrix(m, {get(b + "ffn_down.weight")}, &L.wd, "down weight", e)) return false;
    }
    if (!upload_norm(m, get("output_norm.weight"), &m->out_norm, e)) return false;
    // "output.weight | token_embd.weight" (page "Local inference and
    // architectures", "Rules": this tensor, or that one if it is absent).
    auto it = T.find("output.weight");
    if (it != T.end()) {
        if (!upload_matrix(m, {it->second}, &m->out, "output weight", e)) return false;
    } else {
        m->out = m->embd;
    }

    // cos/sin position cache, computed in f64 and rounded to f32 (section
    // "Memory lifecycle", "Position caches").
    const int64_t hd = c.head_dim;
    const int64_t half = hd / 2;
    m->rope_rows = c.max_ctx;
    std::vector<float> cs(size_t(c.max_ctx * half)), sn(size_t(c.max_ctx * half));
    for (int64_t p = 0; p < c.max_ctx; ++p)
        for (int64_t i = 0; i < half; ++i) {
            const double ang = double(p) * std::pow(c.rope_theta, -2.0 * double(i) / double(hd));
            cs[size_t(p * half + i)] = float(std::cos(ang));
            sn[size_t(p * half + i)] = float(std::sin(ang));
        }
    m->cos_t = static_cast<float*>(dev_alloc(m, cs.size() * 4, "rope cos", e));
    if (!m->cos_t) return false;
    m->sin_t = static_cast<float*>(dev_alloc(m, sn.size() * 4, "rope sin", e));
    if (!m->sin_t) return false;
    if (!check(hipMemcpyAsync(m->cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream),
               "rope cos upload", e))
        return false;
    if (!check(hipMemcpyAsync(m->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, m->stream),
               "rope sin upload", e))
        return false;
    m->cos_l = m->cos_t;
    m->sin_l = m->sin_t;
    if (c.sliding_window > 0 && c.rope_theta_local > 0 && c.rope_theta_local != c.rope_theta) {
        // the local layers' table, built the same way with their theta; the
        // host vectors are refilled only after the first upload has finished
        if (!check(hipStreamSynchronize(m->stream), "rope upload", e)) return false;
        for (int64_t p = 0; p < c.max_ctx; ++p)
            for (int64_t i = 0; i < half; ++i) {
                const double ang = double(p) * std::pow(c.rope_theta_local, -2.0 * double(i) / double(hd));
                cs[size_t(p * half + i)] = float(std::cos(ang));
                sn[size_t(p * half + i)] = float(std::sin(ang));
            }
        m->cos_l = static_cast<float*>(dev_alloc(m, cs.size() * 4, "local rope cos", e));
        if (!m->cos_l) return false;
        m->sin_l = static_cast<float*>(dev_alloc(m, sn.size() * 4, "local rope sin", e));
        if (!m->sin_l) return false;
        if (!check(hipMemcpyAsync(m->cos_l, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream),
                   "local rope cos upload", e) ||
            !check(hipMemcpyAsync(m->sin_l, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, m->stream),
                   "local rope sin upload", e))
            return false;
    }

    m->zeros = static_cast<uint16_t*>(dev_alloc(m, 256, "zero block", e));
    if (!m->zeros) return false;
    if (!check(hipMemsetAsync(m->zeros, 0, 256, m->stream), "zero block init", e)) return false;
    return check(hipStreamSynchronize(m->stream), "upload", e);
}

bool bulk_supported(const df_model* m);

// One conversation's device state (section "Memory lifecycle": the KV cache
// is per conversation, sized to its max context): the KV cache (with its f16
// copies where the bulk-prefill attention reads them), the decode state,
// attention partials, argmax result and generated-token buffer.
bool build_conversation(df_model* m, Fail* e)
{
    const df_config& c = m->cfg;
    const int64_t hd = c.head_dim;
    const size_t kv_elems = size_t(c.n_layers) * size_t(c.n_kv_heads) * size_t(c.max_ctx) * size_t(hd);
    m->kc = static_cast<float*>(dev_alloc(m, kv_elems * 4, "K cache", e));
    if (!m->kc) return false;
    m->vc = static_cast<float*>(dev_alloc(m, kv_elems * 4, "V cache", e));
    if (!m->vc) return false;
    m->kv_bytes = int64_t(kv_elems) * 8;
    if (bulk_supported(m) && kv_shadow_head_dim(int(hd))) {
        // zeroed: a tile's keys past the last written position are read (and
        // weighted by 0), so they must hold finite values
        m->k16 = static_cast<uint16_t*>(dev_alloc(m, kv_elems * 2, "K cache f16 copy", e));
        if (!m->k16) return false;
        m->vt16 = static_cast<uint16_t*>(dev_alloc(m, kv_elems * 2, "V cache f16 copy", e));
        if (!m->vt16) return false;
        if (!check(hipMemsetAsync(m->k16, 0, kv_elems * 2, m->stream), "K copy init", e) ||
            !check(hipMemsetAsync(m->vt16, 0, kv_elems * 2, m->stream), "V copy init", e))
            return false;
        m->kv_bytes += int64_t(kv_elems) * 4;
    }
    m->state = static_cast<DevState*>(dev_alloc(m, sizeof(DevState), "decode state", e));
    if (!m->state) return false;
    const int G = c.n_heads / c.n_kv_heads;
    m->attn_part = static_cast<float*>(dev_alloc(
        m, size_t(c.n_kv_heads) * ATTN_MAX_SPLIT * attn_part_stride(G, int(hd)) * 4, "attention partials", e));
    if (!m->attn_part) return false;
    m->argmax_out = static_cast<int*>(dev_alloc(m, 4, "argmax result", e));
    if (!m->argmax_out) return false;
    if (bulk_supported(m)) {
        // per conversation: two conversations' GEMMs may run at once
        m->gemm_tickets = static_cast<int*>(dev_alloc(m, GEMM_SPLIT_TICKETS * sizeof(int), "GEMM split tickets", e));
        if (!m->gemm_tickets ||
            !check(hipMemsetAsync(m->gemm_tickets, 0, GEMM_SPLIT_TICKETS * sizeof(int), m->stream),
                   "GEMM split tickets init", e))
            return false;
    }
    m->gen_tokens = static_cast<int*>(dev_alloc(m, size_t(c.max_ctx) * 4, "generated tokens", e));
    if (!m->gen_tokens) return false;
    if (!check(hipMemsetAsync(m->state, 0, sizeof(DevState), m->stream), "state init", e)) return false;
    if (!check(hipStreamSynchronize(m->stream), "upload", e)) return false;
    return true;
}

// ---------------------------------------------------------------------------
// The decode step: one token at position kv_len (state->pos), through the
// step list. Per layer: [rms_norm + q/k/v matmul] -> [norm_heads + rope + KV
// append + attention] -> [o matmul + add] -> [rms_norm + gate/up matmul +
// silu + mul] -> [down matmul + add]; then [rms_norm + logits matmul].
// ---------------------------------------------------------------------------
struct StepBufs {
    float *x, *qkv, *att, *mid;
    float* tmp;  // gemma3: o / down output before its rms_norm (d floats)
};

bool step_buffers(df_model* m, StepBufs* b, Fail* e)
{
    const df_config& c = m->cfg;
    const size_t qd = size_t(c.n_heads) * c.head_dim, kvd = size_t(c.n_kv_heads) * c.head_dim;
    b->x = static_cast<float*>(m->pool.alloc(size_t(c.d_model) * 4, USAGE_DEVICE, e));
    b->qkv = static_cast<float*>(m->pool.alloc((qd + 2 * kvd) * 4, USAGE_DEVICE, e));
    b->att = static_cast<float*>(m->pool.alloc(qd * 4, USAGE_DEVICE, e));
    b->mid = static_cast<float*>(m->pool.alloc(size_t(c.ffn_dim) * 4, USAGE_DEVICE, e));
    b->tmp = nullptr;
    if (c.arch == DF_ARCH_GEMMA3) {
        b->tmp = static_cast<float*>(m->pool.alloc(size_t(c.d_model) * 4 + 4, USAGE_DEVICE, e));
        if (!b->tmp) return false;
    }
    return b->x && b->qkv && b->att && b->mid;
}

// Start / end stamps of one launch when its class is being profiled: the
// scope hands an event pair to the launch, which the dispatch stamps.
struct ProfScope {
    df_model* m;
    bool on = false;
    ProfScope(df_model* mm, int kernel) : m(mm)
    {
        if (m->prof_kernel != kernel) return;
        if (m->prof_used == m->prof_events.size()) {
            hipEvent_t a = nullptr, b = nullptr;
            if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
                (void)hipGetLastError();
                return;
            }
            m->prof_events.emplace_back(a, b);
        }
        auto& ev = m->prof_events[m->prof_used++];
        launch_timing() = LaunchTiming{ev.first, ev.second};
        on = true;
    }
    ~ProfScope()
    {
        if (on) launch_timing() = LaunchTiming{};
    }
};

// The launches of one kernel class for layer l of a decode step (layer is
// ignored for embed / logits / argmax).
hipError_t launch_class(df_model* m, const StepBufs& b, int kernel, int l, int grid_splits,
                        float* logits)
{
    const df_config& c = m->cfg;
    const float eps = float(c.rms_eps);
    const int hd = c.head_dim;
    const int64_t qd = int64_t(c.n_heads) * hd, kvd = int64_t(c.n_kv_heads) * hd;
    const size_t kv_layer = size_t(c.n_kv_heads) * size_t(c.max_ctx) * size_t(hd);
    const Layer* L = (l >= 0 && l < c.n_layers) ? &m->layers[size_t(l)] : nullptr;
    AttnDecodeArgs a{};
    if (L) {
        a.qkv = b.qkv;
        a.q_norm = L->q_norm;
        a.k_norm = L->k_norm;
        a.bias = L->bqkv;
        a.eps = eps;
        a.adjacent = c.rope_pairing == DF_ROPE_ADJACENT;
        a.cos_t = L->local ? m->cos_l : m->cos_t;
        a.sin_t = L->local ? m->sin_l : m->sin_t;
        a.window = L->local ? c.sliding_window : 0;
        a.kc = m->kc + size_t(l) * kv_layer;
        a.vc = m->vc + size_t(l) * kv_layer;
        a.k16 = m->k16 ? m->k16 + size_t(l) * kv_layer : nullptr;
        a.vt16 = m->vt16 ? m->vt16 + size_t(l) * kv_layer : nullptr;
        a.max_ctx = c.max_ctx;
        a.n_heads = c.n_heads;
        a.n_kv = c.n_kv_heads;
        a.head_dim = hd;
        a.state_pos = &m->state->pos;
        a.part = m->attn_part;
        a.out = b.att;
        a.grid_splits = grid_splits;
    }
    const bool gemma = c.arch == DF_ARCH_GEMMA3;
    // gemma3: the matmul output goes to tmp and its rms_norm is added to x
    // by a second launch; both count as one launch of the class.
    auto norm_added = [&](const Weight& W, const float* in, const float* post_w) {
        const LaunchTiming saved = launch_timing();
        launch_timing() = LaunchTiming{saved.start, nullptr};
        hipError_t r = launch_matvec(W, MV_STORE, in, nullptr, eps, c.d_model, 0, b.tmp, m->stream);
        launch_timing() = LaunchTiming{nullptr, saved.stop};
        if (r == hipSuccess) r = launch_norm_add_rows(b.x, b.tmp, post_w, 1, c.d_model, eps, m->stream);
        launch_timing() = saved;
        return r;
    };
    switch (kernel) {
    case DF_K_EMBED:
        return launch_embed(m->embd, nullptr, &m->state->tok, 1, b.x, m->stream, embed_scale(c));
    case DF_K_QKV: return launch_matvec(L->wqkv, MV_STORE, b.x, L->attn_norm, eps, qd + 2 * kvd, 0, b.qkv, m->stream);
    case DF_K_ATTN: return launch_attn_decode(a, m->stream);
    case DF_K_ATTN_MERGE: return launch_attn_combine(a, m->stream);
    case DF_K_O:
        if (gemma) return norm_added(L->wo, b.att, L->post_attn_norm);
        return launch_matvec(L->wo, MV_RESID, b.att, nullptr, eps, c.d_model, 0, b.x, m->stream);
    case DF_K_GATE_UP:
        return launch_matvec(L->wgu, MV_SWIGLU, b.x, L->ffn_norm, eps, c.ffn_dim, c.ffn_dim, b.mid, m->stream,
                             gemma ? ACT_GELU_TANH : ACT_SILU);
    case DF_K_DOWN:
        if (gemma) return norm_added(L->wd, b.mid, L->post_ffn_norm);
        return launch_matvec(L->wd, MV_RESID, b.mid, nullptr, eps, c.d_model, 0, b.x, m->stream);
    case DF_K_LOGITS: return launch_matvec(m->out, MV_STORE, b.x, m->out_norm, eps, c.vocab, 0, logits, m->stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_step(df_model* m, const StepBufs& b, int grid_splits, float* logits)
{
    static const int per_layer[] = {DF_K_QKV, DF_K_ATTN, DF_K_ATTN_MERGE, DF_K_O, DF_K_GATE_UP, DF_K_DOWN};
    hipError_t r;
    {
        ProfScope ps(m, DF_K_EMBED);
        r = launch_class(m, b, DF_K_EMBED, -1, grid_splits, logits);
    }
    for (int l = 0; l < m->cfg.n_layers && r == hipSuccess; ++l) {
        for (int k : per_layer) {
            ProfScope ps(m, k);
            r = launch_class(m, b, k, l, grid_splits, logits);
            if (r != hipSuccess) break;
        }
    }
    if (r == hipSuccess && logits) {
        ProfScope ps(m, DF_K_LOGITS);
        r = launch_class(m, b, DF_K_LOGITS, -1, grid_splits, logits);
    }
    return r;
}

struct BusyGuard {
    df_model* m;
    bool ok;
    explicit BusyGuard(df_model* mm) : m(mm)
    {
        int expect = 0;
        ok = m->busy.compare_exchange_strong(expect, 1);
    }
    ~BusyGuard()
    {
        if (ok) m->busy.store(0);
    }
};

df_status set_err(df_model* m, df_status code, const std::string& msg)
{
    m->err = msg;
    return code;
}

void collect_event_time(df_model* m)
{
    if (!m->ev_kind) return;
    if (hipEventSynchronize(m->ev1) == hipSuccess) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, m->ev0, m->ev1) == hipSuccess) {
            if (m->ev_kind == 1) m->last_step_ms = ms;
            else m->last_prefill_ms = ms;
        }
    }
    (void)hipGetLastError();
    m->ev_kind = 0;
}

df_status decode_one(df_model* m, int32_t tok, float* logits)
{
    Fail e{DF_OK, ""};
    const int pos = m->kv_len;
    m->pool.reset();
    StepBufs b{};
    if (!step_buffers(m, &b, &e)) return set_err(m, e.code, e.msg);
    hipError_t r = launch_set_state(m->state, pos, tok, 0, m->stream);
    if (r == hipSuccess) r = launch_step(m, b, attn_splits(pos), logits);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("decode launch failed: %s", hipGetErrorString(r)));
    }
    m->kv_len = pos + 1;
    return DF_OK;
}

// ---------------------------------------------------------------------------
// Bulk prefill: n tokens at positions kv_len .. kv_len+n-1 in one pass of
// the step list over n rows (page "Execution contract", "Forward phase":
// bulk prefill must match token-by-token within epsilon). Per layer:
// [rms_norm rows -> f16] [q/k/v GEMM] [norm_heads + rope + KV append]
// [causal flash attention] [o GEMM + add] [rms_norm rows -> f16]
// [gate/up GEMM + silu * up] [down GEMM + add]; then the last row's
// [rms_norm + logits matvec]. Needs f16 or 8-bit block weights (8-bit
// blocks are dequantised to f16 inside the GEMM's weight load path).
// ---------------------------------------------------------------------------
bool bulk_supported(const df_model* m)
{
    return m->cfg.n_layers == 0 || m->layers[0].wqkv.dtype == W_F16 || m->layers[0].wqkv.dtype == W_Q8;
}

// Bulk prefill activations for S rows.
struct PfBufs {
    float* x;          // [S][d] residual stream
    uint16_t* h16;     // [S][d] normed rows, f16
    float* qkv;        // [S][qd + 2 kvd]
    uint16_t* q16;     // [S][qd] q after rope, f16
    uint16_t* att16;   // [S][qd] attention output, f16
    uint16_t* mid16;   // [S][F] gated FFN activation, f16
    float* tmp;        // gemma3: [S][d] o / down outputs before their rms_norm
    int* toks;         // [S]
    uint16_t* wdq;     // 8-bit weights, S >= PF_DEQUANT_MIN_ROWS: one matrix dequantised to f16
    float* gws;        // partial sums of split GEMM tiles (null when no GEMM splits)
};

bool pf_buffers(df_model* m, int S, PfBufs* b, Fail* e)
{
    const df_config& c = m->cfg;
    const size_t d = size_t(c.d_model), F = size_t(c.ffn_dim);
    const size_t qd = size_t(c.n_heads) * c.head_dim, kvd = size_t(c.n_kv_heads) * c.head_dim;
    auto A = [&](size_t bytes) { return m->pool.alloc(bytes, USAGE_DEVICE, e); };
    b->x = static_cast<float*>(A(size_t(S) * d * 4));
    b->h16 = static_cast<uint16_t*>(A(size_t(S) * d * 2));
    b->qkv = static_cast<float*>(A(size_t(S) * (qd + 2 * kvd) * 4));
    b->q16 = static_cast<uint16_t*>(A(size_t(S) * qd * 2));
    b->att16 = static_cast<uint16_t*>(A(size_t(S) * qd * 2));
    b->mid16 = static_cast<uint16_t*>(A(size_t(S) * F * 2));
    b->toks = static_cast<int*>(A(size_t(S) * 4));
    b->tmp = c.arch == DF_ARCH_GEMMA3 ? static_cast<float*>(A(size_t(S) * d * 4)) : nullptr;
    b->wdq = nullptr;
    b->gws = nullptr;
    if (c.n_layers > 0) {
        // the largest partial-sum space of the four GEMMs (as planned for S rows)
        const bool q8_in_gemm = m->layers[0].wqkv.scales && S < PF_DEQUANT_MIN_ROWS;
        const bool gemma = c.arch == DF_ARCH_GEMMA3;
        const int64_t N[4] = {int64_t(qd + 2 * kvd), int64_t(d), int64_t(F), int64_t(d)};
        const int64_t K[4] = {int64_t(d), int64_t(qd), int64_t(d), int64_t(F)};
        const int mode[4] = {GEMM_STORE_F32, gemma ? GEMM_STORE_F32 : GEMM_ADD_F32, GEMM_SWIGLU_F16,
                             gemma ? GEMM_STORE_F32 : GEMM_ADD_F32};
        size_t ws = 0;
        for (int i = 0; i < 4; ++i)
            ws = std::max(ws, gemm_split_ws_bytes(S, N[i], K[i], i == 2 ? int64_t(F) : 0, mode[i], q8_in_gemm));
        if (ws) {
            b->gws = static_cast<float*>(A(ws));
            if (!b->gws) return false;
        }
    }
    if (c.n_layers > 0 && m->layers[0].wqkv.scales && S >= PF_DEQUANT_MIN_ROWS) {
        const size_t most = std::max(std::max((qd + 2 * kvd) * d, d * qd), std::max(2 * F * d, d * F));
        b->wdq = static_cast<uint16_t*>(A(most * 2));
        if (!b->wdq) return false;
    }
    return b->x && b->h16 && b->qkv && b->q16 && b->att16 && b->mid16 && b->toks &&
           (c.arch != DF_ARCH_GEMMA3 || b->tmp);
}

// The bulk-prefill launches of layer l for S rows at positions p0.., one
// class at a time (the classes in step-list order):
//   DF_K_PF_QKV     rms_norm rows -> f16, q/k/v GEMM
//   DF_K_PF_ROWS    bias + norm_heads + rope + KV append (+ the f16 copies)
//   DF_K_PF_ATTN    causal attention
//   DF_K_PF_O       o GEMM + residual add (gemma3: + rms_norm of o)
//   DF_K_PF_GATE_UP rms_norm rows -> f16, gate/up GEMM + gate activation * up
//   DF_K_PF_DOWN    down GEMM + residual add (gemma3: + rms_norm of down)
hipError_t pf_launch(df_model* m, const PfBufs& b, int kernel, int l, int S, int p0)
{
    const df_config& c = m->cfg;
    const Layer& L = m->layers[size_t(l)];
    const int d = c.d_model, hd = c.head_dim, F = c.ffn_dim;
    const int qd = c.n_heads * hd, kvd = c.n_kv_heads * hd;
    const float eps = float(c.rms_eps);
    const bool gemma = c.arch == DF_ARCH_GEMMA3;
    const size_t kv_layer = size_t(c.n_kv_heads) * size_t(c.max_ctx) * size_t(hd);
    GemmArgs g{};
    g.zeros = m->zeros;
    g.ws = b.gws;
    g.tickets = m->gemm_tickets;
    g.M = S;
    hipError_t r = hipSuccess;
    // The GEMM's B operand: the weight as stored, or (8-bit blocks with a
    // dequantisation buffer) its f16 rows converted just before the GEMM.
    auto weights = [&](const Weight& W) {
        g.B = static_cast<const uint16_t*>(W.data);
        g.Bsc = W.scales;
        if (r == hipSuccess && W.scales && b.wdq) {
            r = launch_dequant_q8(W.data, W.scales, W.rows, W.cols, b.wdq, m->stream);
            g.B = b.wdq;
            g.Bsc = nullptr;
        }
    };
    switch (kernel) {
    case DF_K_PF_QKV:
        r = launch_rmsnorm_rows(b.x, L.attn_norm, S, d, eps, b.h16, m->stream);
        g.A = b.h16; g.lda = d;
        weights(L.wqkv); g.ldb = d;
        g.C = b.qkv; g.ldc = qd + 2 * kvd; g.N = qd + 2 * kvd; g.K = d;
        if (r == hipSuccess) r = launch_gemm(g, GEMM_STORE_F32, m->stream);
        return r;
    case DF_K_PF_ROWS: {
        QkPostArgs qa{};
        qa.qkv = b.qkv; qa.q_norm = L.q_norm; qa.k_norm = L.k_norm; qa.eps = eps;
        qa.bias = L.bqkv; qa.adjacent = c.rope_pairing == DF_ROPE_ADJACENT;
        qa.cos_t = L.local ? m->cos_l : m->cos_t; qa.sin_t = L.local ? m->sin_l : m->sin_t;
        qa.kc = m->kc + size_t(l) * kv_layer; qa.vc = m->vc + size_t(l) * kv_layer;
        qa.q16 = b.q16; qa.S = S; qa.p0 = p0; qa.n_heads = c.n_heads; qa.n_kv = c.n_kv_heads;
        qa.head_dim = hd; qa.max_ctx = c.max_ctx;
        r = launch_qk_post_rows(qa, m->stream);
        if (r != hipSuccess || !m->k16) return r;
        // the f16 copies of the rows just appended
        KvShadowArgs ka{};
        ka.kc = qa.kc; ka.vc = qa.vc;
        ka.k16 = m->k16 + size_t(l) * kv_layer;
        ka.vt16 = m->vt16 + size_t(l) * kv_layer;
        ka.pos0 = p0; ka.n = S; ka.n_kv = c.n_kv_heads; ka.head_dim = hd; ka.max_ctx = c.max_ctx;
        ka.do_k = ka.do_v = 1;
        return launch_kv_shadow(ka, m->stream);
    }
    case DF_K_PF_ATTN: {
        AttnPrefillArgs aa{};
        aa.k16 = m->k16 ? m->k16 + size_t(l) * kv_layer : nullptr;
        aa.vt16 = m->vt16 ? m->vt16 + size_t(l) * kv_layer : nullptr;
        aa.q16 = b.q16; aa.kc = m->kc + size_t(l) * kv_layer; aa.vc = m->vc + size_t(l) * kv_layer;
        aa.out16 = b.att16;
        aa.S = S; aa.p0 = p0; aa.n_heads = c.n_heads; aa.n_kv = c.n_kv_heads;
        aa.head_dim = hd; aa.max_ctx = c.max_ctx;
        aa.window = L.local ? c.sliding_window : 0;
        return launch_attn_prefill(aa, m->stream);
    }
    case DF_K_PF_O:
        g.A = b.att16; g.lda = qd;
        weights(L.wo); g.ldb = qd;
        g.C = gemma ? static_cast<void*>(b.tmp) : b.x; g.ldc = d; g.N = d; g.K = qd;
        if (r == hipSuccess) r = launch_gemm(g, gemma ? GEMM_STORE_F32 : GEMM_ADD_F32, m->stream);
        if (r == hipSuccess && gemma) r = launch_norm_add_rows(b.x, b.tmp, L.post_attn_norm, S, d, eps, m->stream);
        return r;
    case DF_K_PF_GATE_UP:
        r = launch_rmsnorm_rows(b.x, L.ffn_norm, S, d, eps, b.h16, m->stream);
        g.A = b.h16; g.lda = d;
        weights(L.wgu); g.ldb = d;
        g.C = b.mid16; g.ldc = F; g.N = F; g.K = d; g.up_rows = F;
        g.act = gemma ? ACT_GELU_TANH : ACT_SILU;
        if (r == hipSuccess) r = launch_gemm(g, GEMM_SWIGLU_F16, m->stream);
        return r;
    case DF_K_PF_DOWN:
        g.A = b.mid16; g.lda = F;
        weights(L.wd); g.ldb = F;
        g.C = gemma ? static_cast<void*>(b.tmp) : b.x; g.ldc = d; g.N = d; g.K = F;
        if (r == hipSuccess) r = launch_gemm(g, gemma ? GEMM_STORE_F32 : GEMM_ADD_F32, m->stream);
        if (r == hipSuccess && gemma) r = launch_norm_add_rows(b.x, b.tmp, L.post_ffn_norm, S, d, eps, m->stream);
        return r;
    }
    return hipErrorInvalidValue;
}

df_status prefill(df_model* m, const int32_t* tokens, int32_t n, float* logits)
{
    const df_config& c = m->cfg;
    Fail e{DF_OK, ""};
    const int S = n, p0 = m->kv_len;
    m->pool.reset();
    PfBufs b{};
    if (!pf_buffers(m, S, &b, &e)) return set_err(m, e.code, e.msg);
    static const int classes[] = {DF_K_PF_QKV, DF_K_PF_ROWS, DF_K_PF_ATTN, DF_K_PF_O, DF_K_PF_GATE_UP,
                                  DF_K_PF_DOWN};
    hipError_t r = hipMemcpyAsync(b.toks, tokens, size_t(S) * 4, hipMemcpyHostToDevice, m->stream);
    if (r == hipSuccess) r = launch_embed(m->embd, b.toks, nullptr, S, b.x, m->stream, embed_scale(c));
    for (int l = 0; l < c.n_layers && r == hipSuccess; ++l)
        for (int k : classes) {
            r = pf_launch(m, b, k, l, S, p0);
            if (r != hipSuccess) break;
        }
    if (r == hipSuccess && logits)
        r = launch_matvec(m->out, MV_STORE, b.x + size_t(S - 1) * c.d_model, m->out_norm,
                          float(c.rms_eps), c.vocab, 0, logits, m->stream);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("bulk prefill launch failed: %s", hipGetErrorString(r)));
    }
    m->kv_len = p0 + S;
    return DF_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

df_status df_load(const df_config* cfg, const df_tensor* tensors, size_t n_tensors,
                  const df_options* opt, df_model** out)
{
    const auto t_start = std::chrono::steady_clock::now();
    g_load_error.clear();
    if (!out) {
        g_load_error = "df_load: out is NULL";
        return DF_ERR_INVALID_ARGUMENT;
    }
    *out = nullptr;
    Fail e{DF_OK, ""};
    if (opt && opt->flags) {
        g_load_error = fmt("df_load: option flags 0x%x: none are defined", unsigned(opt->flags));
        return DF_ERR_INVALID_ARGUMENT;
    }
    std::map<std::string, const df_tensor*> found;
    if (!validate_config(cfg, &e) || !validate_tensors(cfg, tensors, n_tensors, &found, &e)) {
        g_load_error = e.msg;
        return e.code;
    }

    // Backend init: the first device call.
    int ndev = 0;
    hipError_t r = hipGetDeviceCount(&ndev);
    if (r != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        g_load_error = fmt("backend init: no HIP device (%s)",
                           r != hipSuccess ? hipGetErrorString(r) : "0 devices");
        return DF_ERR_BACKEND_INIT;
    }
    const int dev = opt ? opt->device : 0;
    if (dev < 0 || dev >= ndev) {
        g_load_error = fmt("backend init: device %d out of range (0..%d)", dev, ndev - 1);
        return DF_ERR_BACKEND_INIT;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        g_load_error = "backend init: hipGetDeviceProperties failed";
        return DF_ERR_BACKEND_INIT;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        g_load_error = fmt("backend init: device %d is %s; this library is built for gfx950",
                           dev, prop.gcnArchName);
        return DF_ERR_BACKEND_INIT;
    }
    if (hipSetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        g_load_error = fmt("backend init: hipSetDevice(%d) failed", dev);
        return DF_ERR_BACKEND_INIT;
    }
    if (!noalloc_scratch_init(dev, &g_load_error)) return DF_ERR_BACKEND_INIT;

    df_model* m = new (std::nothrow) df_model();
    if (!m) {
        g_load_error = "host allocation of the model failed";
        return DF_ERR_OUT_OF_MEMORY;
    }
    m->cfg = *cfg;
    m->device = dev;
    if (opt && opt->stream) {
        m->stream = static_cast<hipStream_t>(opt->stream);
    } else {
        if (hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking) != hipSuccess) {
            (void)hipGetLastError();
            delete m;
            g_load_error = "backend init: hipStreamCreate failed";
            return DF_ERR_BACKEND_INIT;
        }
        m->own_stream = true;
    }
    if (hipEventCreate(&m->ev0) != hipSuccess || hipEventCreate(&m->ev1) != hipSuccess) {
        (void)hipGetLastError();
        release(m);
        delete m;
        g_load_error = "backend init: hipEventCreate failed";
        return DF_ERR_BACKEND_INIT;
    }
    m->wstore = std::make_shared<WeightStore>();
    m->wstore->device = dev;
    m->alloc_to = &m->wstore->allocs;
    const bool weights_ok = build_weights(m, found, &e);
    m->alloc_to = nullptr;
    if (!weights_ok || !build_conversation(m, &e)) {
        release(m);
        delete m;
        g_load_error = e.msg;
        return e.code;
    }
    m->load_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
    *out = m;
    return DF_OK;
}

df_status df_session(const df_model* base, int32_t max_ctx, const df_options* opt, df_model** out)
{
    const auto t_start = std::chrono::steady_clock::now();
    g_load_error.clear();
    if (!out) {
        g_load_error = "df_session: out is NULL";
        return DF_ERR_INVALID_ARGUMENT;
    }
    *out = nullptr;
    if (!base) {
        g_load_error = "df_session: model is NULL";
        return DF_ERR_INVALID_ARGUMENT;
    }
    if (max_ctx < 1 || max_ctx > base->rope_rows) {
        g_load_error = fmt("df_session: max_ctx = %d: expected 1..%d (the positions the model's "
                           "cos/sin table covers)", max_ctx, base->rope_rows);
        return DF_ERR_INVALID_ARGUMENT;
    }
    if (opt && opt->flags) {
        g_load_error = fmt("df_session: option flags 0x%x: none are defined", unsigned(opt->flags));
        return DF_ERR_INVALID_ARGUMENT;
    }
    if (hipSetDevice(base->device) != hipSuccess) {
        (void)hipGetLastError();
        g_load_error = fmt("df_session: hipSetDevice(%d) failed", base->device);
        return DF_ERR_DEVICE;
    }
    df_model* m = new (std::nothrow) df_model();
    if (!m) {
        g_load_error = "host allocation of the session failed";
        return DF_ERR_OUT_OF_MEMORY;
    }
    m->cfg = base->cfg;
    m->cfg.max_ctx = max_ctx;
    m->device = base->device;
    m->wstore = base->wstore;
    m->weight_bytes = base->weight_bytes;
    m->rope_rows = base->rope_rows;
    m->embd = base->embd;
    m->out = base->out;
    m->out_norm = base->out_norm;
    m->layers = base->layers;
    m->cos_t = base->cos_t;
    m->sin_t = base->sin_t;
    m->cos_l = base->cos_l;
    m->sin_l = base->sin_l;
    m->zeros = base->zeros;
    Fail e{DF_OK, ""};
    bool ok = true;
    if (opt && opt->stream) {
        m->stream = static_cast<hipStream_t>(opt->stream);
    } else {
        ok = check(hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking), "session stream", &e,
                   DF_ERR_DEVICE);
        m->own_stream = ok;
    }
    ok = ok && check(hipEventCreate(&m->ev0), "session events", &e, DF_ERR_DEVICE) &&
         check(hipEventCreate(&m->ev1), "session events", &e, DF_ERR_DEVICE) &&
         build_conversation(m, &e);
    if (!ok) {
        release(m);
        delete m;
        g_load_error = e.msg;
        return e.code;
    }
    m->load_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
    *out = m;
    return DF_OK;
}

df_status df_forward(df_model* m, const int32_t* tokens, int32_t n, float* logits_dev)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    if (!tokens || n <= 0)
        return set_err(m, DF_ERR_INVALID_ARGUMENT, fmt("df_forward: tokens %s, n = %d",
                                                       tokens ? "given" : "NULL", n));
    if (int64_t(m->kv_len) + n > m->cfg.max_ctx)
        return set_err(m, DF_ERR_CONTEXT_FULL,
                       fmt("df_forward: %d positions in the cache + %d new > max_ctx %d",
                           m->kv_len, n, m->cfg.max_ctx));
    for (int32_t i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= m->cfg.vocab)
            return set_err(m, DF_ERR_INVALID_ARGUMENT,
                           fmt("df_forward: token %d at index %d outside [0, %d)", tokens[i], i,
                               m->cfg.vocab));
    if (hipSetDevice(m->device) != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, "hipSetDevice failed");
    }
    collect_event_time(m);
    (void)hipEventRecord(m->ev0, m->stream);
    df_status st = DF_OK;
    if (n > 1 && bulk_supported(m)) {
        st = prefill(m, tokens, n, logits_dev);
    } else {
        // One token, or block weights the matrix-core path does not take
        // (f32): the decode kernels, one position after another.
        for (int32_t i = 0; i < n && st == DF_OK; ++i)
            st = decode_one(m, tokens[i], i == n - 1 ? logits_dev : nullptr);
    }
    (void)hipEventRecord(m->ev1, m->stream);
    m->ev_kind = n == 1 ? 1 : 2;
    if (st == DF_OK) m->n_forward++;
    return st;
}

df_status df_forward_noalloc(df_model* m, const int32_t* tokens, int32_t n, float* logits_dev)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    const df_config& c = m->cfg;
    if (!tokens || n <= 0)
        return set_err(m, DF_ERR_INVALID_ARGUMENT, fmt("df_forward_noalloc: tokens %s, n = %d",
                                                       tokens ? "given" : "NULL", n));
    if (int64_t(m->kv_len) + n > c.max_ctx)
        return set_err(m, DF_ERR_CONTEXT_FULL,
                       fmt("df_forward_noalloc: %d positions in the cache + %d new > max_ctx %d",
                           m->kv_len, n, c.max_ctx));
    for (int32_t i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= c.vocab)
            return set_err(m, DF_ERR_INVALID_ARGUMENT,
                           fmt("df_forward_noalloc: token %d at index %d outside [0, %d)", tokens[i], i,
                               c.vocab));
    if (m->prof_kernel >= 0)
        return set_err(m, DF_ERR_INVALID_ARGUMENT,
                       "df_forward_noalloc: a kernel class is being profiled (df_profile), which creates "
                       "events; turn profiling off first");
    // The step's activations, each 256-byte aligned, carved from the fixed array.
    const size_t qd = size_t(c.n_heads) * c.head_dim, kvd = size_t(c.n_kv_heads) * c.head_dim;
    const bool gemma = c.arch == DF_ARCH_GEMMA3;
    auto up = [](size_t bytes) { return (bytes + 255) & ~size_t(255); };
    const size_t sizes[5] = {size_t(c.d_model) * 4, (qd + 2 * kvd) * 4, qd * 4, size_t(c.ffn_dim) * 4,
                             gemma ? size_t(c.d_model) * 4 + 4 : 0};
    size_t need = 0;
    for (size_t b : sizes) need += up(b);
    if (need > NOALLOC_SCRATCH_BYTES)
        return set_err(m, DF_ERR_UNSUPPORTED_OP,
                       fmt("df_forward_noalloc: the decode step's activations take %zu bytes (d_model %d, "
                           "q|k|v %zu, attention %zu, ffn %d floats); the fixed array holds %zu",
                           need, c.d_model, qd + 2 * kvd, qd, c.ffn_dim, NOALLOC_SCRATCH_BYTES));
    char* base = static_cast<char*>(noalloc_scratch(m->device));
    if (!base)
        return set_err(m, DF_ERR_DEVICE, fmt("df_forward_noalloc: no fixed array address for device %d",
                                             m->device));
    StepBufs b{};
    size_t off = 0;
    float* parts[5];
    for (int i = 0; i < 5; ++i) {
        parts[i] = sizes[i] ? reinterpret_cast<float*>(base + off) : nullptr;
        off += up(sizes[i]);
    }
    b.x = parts[0];
    b.qkv = parts[1];
    b.att = parts[2];
    b.mid = parts[3];
    b.tmp = parts[4];
    if (hipSetDevice(m->device) != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, "hipSetDevice failed");
    }
    collect_event_time(m);
    (void)hipEventRecord(m->ev0, m->stream);
    // Token by token through the decode kernels (separate launches), the
    // same launches df_forward makes for one token.
    hipError_t r = hipSuccess;
    int32_t done = 0;
    for (; done < n && r == hipSuccess; ++done) {
        const int pos = m->kv_len + done;
        r = launch_set_state(m->state, pos, tokens[done], 0, m->stream);
        if (r == hipSuccess) r = launch_step(m, b, attn_splits(pos), done == n - 1 ? logits_dev : nullptr);
    }
    if (r != hipSuccess) {
        (void)hipGetLastError();
        m->kv_len += done - 1;  // the failed step's position was not completed
        return set_err(m, DF_ERR_DEVICE, fmt("df_forward_noalloc: launch failed: %s", hipGetErrorString(r)));
    }
    (void)hipEventRecord(m->ev1, m->stream);
    m->ev_kind = n == 1 ? 1 : 2;
    m->kv_len += n;
    m->n_forward++;
    return DF_OK;
}

df_status df_generate(df_model* m, int32_t first_token, int32_t n_steps, int32_t* tokens_dev,
                      float* logits_dev)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    if (n_steps <= 0 || !tokens_dev)
        return set_err(m, DF_ERR_INVALID_ARGUMENT, "df_generate: n_steps <= 0 or tokens_dev NULL");
    if (first_token < 0 || first_token >= m->cfg.vocab)
        return set_err(m, DF_ERR_INVALID_ARGUMENT,
                       fmt("df_generate: first token %d outside [0, %d)", first_token, m->cfg.vocab));
    if (int64_t(m->kv_len) + n_steps > m->cfg.max_ctx)
        return set_err(m, DF_ERR_CONTEXT_FULL,
                       fmt("df_generate: %d positions + %d steps > max_ctx %d", m->kv_len, n_steps,
                           m->cfg.max_ctx));
    if (hipSetDevice(m->device) != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, "hipSetDevice failed");
    }
    collect_event_time(m);
    Fail e{DF_OK, ""};
    m->pool.reset();
    StepBufs b{};
    if (!step_buffers(m, &b, &e)) return set_err(m, e.code, e.msg);
    float* lg = static_cast<float*>(m->pool.alloc(size_t(m->cfg.vocab) * 4, USAGE_DEVICE, &e));
    if (!lg) return set_err(m, e.code, e.msg);
    hipError_t r = launch_set_state(m->state, m->kv_len, first_token, 0, m->stream);
    // One decode step + greedy argmax, position and token read from device
    // state: the same launches serve every step, so they are captured into a
    // graph once and replayed (unless a kernel class is being profiled).
    const int max_splits = attn_splits(m->cfg.max_ctx - 1);
    auto step_launches = [&]() -> hipError_t {
        hipError_t rr = launch_step(m, b, max_splits, lg);
        if (rr == hipSuccess) {
            ProfScope ps(m, DF_K_ARGMAX);
            rr = launch_argmax(lg, m->cfg.vocab, m->state, m->argmax_out, 1, m->gen_tokens, m->stream);
        }
        return rr;
    };
    const std::vector<void*> key{b.x, b.qkv, b.att, b.mid, lg};
    const bool use_graph = m->prof_kernel < 0;
    if (use_graph && (!m->gen_exec || m->gen_key != key) && r == hipSuccess) {
        if (m->gen_exec) {
            (void)hipGraphExecDestroy(m->gen_exec);
            m->gen_exec = nullptr;
        }
        hipGraph_t graph = nullptr;
        hipError_t c = hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal);
        if (c == hipSuccess) {
            const hipError_t launched = step_launches();
            c = hipStreamEndCapture(m->stream, &graph);
            if (c == hipSuccess && launched != hipSuccess) c = launched;
        }
        if (c == hipSuccess) c = hipGraphInstantiate(&m->gen_exec, graph, nullptr, nullptr, 0);
        if (graph) (void)hipGraphDestroy(graph);
        if (c != hipSuccess) {
            (void)hipGetLastError();
            m->gen_exec = nullptr;
        } else {
            m->gen_key = key;
        }
    }
    for (int32_t i = 0; i < n_steps && r == hipSuccess; ++i) {
        if (use_graph && m->gen_exec) r = hipGraphLaunch(m->gen_exec, m->stream);
        else r = step_launches();
    }
    if (r == hipSuccess)
        r = hipMemcpyAsync(tokens_dev, m->gen_tokens, size_t(n_steps) * 4, hipMemcpyDeviceToDevice,
                           m->stream);
    if (r == hipSuccess && logits_dev)
        r = hipMemcpyAsync(logits_dev, lg, size_t(m->cfg.vocab) * 4, hipMemcpyDeviceToDevice, m->stream);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("df_generate: launch failed: %s", hipGetErrorString(r)));
    }
    m->kv_len += n_steps;
    m->n_forward += n_steps;
    return DF_OK;
}

df_status df_reset_kv_cache(df_model* m)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    m->kv_len = 0;
    return DF_OK;
}

void df_free(df_model** pm)
{
    if (!pm || !*pm) return;
    df_model* m = *pm;
    (void)hipSetDevice(m->device);
    release(m);
    delete m;
    *pm = nullptr;
}

const char* df_last_error(const df_model* m)
{
    return m ? m->err.c_str() : g_load_error.c_str();
}

df_status df_get_timings(df_model* m, df_timings* out)
{
    if (!m || !out) return DF_ERR_INVALID_ARGUMENT;
    (void)hipSetDevice(m->device);
    (void)hipStreamSynchronize(m->stream);
    collect_event_time(m);
    out->load_ms = m->load_ms;
    out->last_prefill_ms = m->last_prefill_ms;
    out->last_step_ms = m->last_step_ms;
    out->n_forward = m->n_forward;
    out->weight_bytes = m->weight_bytes;
    out->kv_bytes = m->kv_bytes;
    out->pool_bytes = int64_t(m->pool.bytes());
    return DF_OK;
}

df_status df_kv_length(const df_model* m, int32_t* out)
{
    if (!m || !out) return DF_ERR_INVALID_ARGUMENT;
    *out = m->kv_len;
    return DF_OK;
}

df_status df_argmax(df_model* m, const float* logits_dev, int32_t* token_host)
{
    if (!m || !logits_dev || !token_host) return DF_ERR_INVALID_ARGUMENT;
    (void)hipSetDevice(m->device);
    hipError_t r = launch_argmax(logits_dev, m->cfg.vocab, m->state, m->argmax_out, 0, nullptr, m->stream);
    if (r == hipSuccess)
        r = hipMemcpyAsync(token_host, m->argmax_out, 4, hipMemcpyDeviceToHost, m->stream);
    if (r == hipSuccess) r = hipStreamSynchronize(m->stream);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("df_argmax: %s", hipGetErrorString(r)));
    }
    return DF_OK;
}

static df_status kv_copy(df_model* m, int32_t layer, int32_t which, int32_t pos0, int32_t n,
                         float* host, bool to_host)
{
    const df_config& c = m->cfg;
    if (layer < 0 || layer >= c.n_layers || (which != 0 && which != 1) || pos0 < 0 || n < 0 ||
        int64_t(pos0) + n > c.max_ctx || (!host && n > 0))
        return set_err(m, DF_ERR_INVALID_ARGUMENT,
                       fmt("kv rows: layer %d which %d rows [%d, %d) out of range", layer, which,
                           pos0, pos0 + n));
    (void)hipSetDevice(m->device);
    float* base = (which ? m->vc : m->kc) +
                  size_t(layer) * size_t(c.n_kv_heads) * size_t(c.max_ctx) * size_t(c.head_dim);
    for (int g = 0; g < c.n_kv_heads && n > 0; ++g) {
        float* dev = base + (size_t(g) * c.max_ctx + size_t(pos0)) * c.head_dim;
        float* h = host + size_t(g) * n * c.head_dim;
        const size_t bytes = size_t(n) * c.head_dim * 4;
        hipError_t r = to_host ? hipMemcpyAsync(h, dev, bytes, hipMemcpyDeviceToHost, m->stream)
                               : hipMemcpyAsync(dev, h, bytes, hipMemcpyHostToDevice, m->stream);
        if (r != hipSuccess) {
            (void)hipGetLastError();
            return set_err(m, DF_ERR_DEVICE, fmt("kv copy: %s", hipGetErrorString(r)));
        }
    }
    if (!to_host && m->k16 && n > 0) {
        // keep the f16 copies of the written rows current
        const size_t kv_layer = size_t(c.n_kv_heads) * size_t(c.max_ctx) * size_t(c.head_dim);
        KvShadowArgs ka{};
        ka.kc = m->kc + size_t(layer) * kv_layer;
        ka.vc = m->vc + size_t(layer) * kv_layer;
        ka.k16 = m->k16 + size_t(layer) * kv_layer;
        ka.vt16 = m->vt16 + size_t(layer) * kv_layer;
        ka.pos0 = pos0; ka.n = n; ka.n_kv = c.n_kv_heads; ka.head_dim = c.head_dim; ka.max_ctx = c.max_ctx;
        ka.do_k = which == 0;
        ka.do_v = which == 1;
        hipError_t r = launch_kv_shadow(ka, m->stream);
        if (r != hipSuccess) {
            (void)hipGetLastError();
            return set_err(m, DF_ERR_DEVICE, fmt("kv copy: %s", hipGetErrorString(r)));
        }
    }
    if (hipStreamSynchronize(m->stream) != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, "kv copy: synchronise failed");
    }
    return DF_OK;
}

df_status df_read_kv(df_model* m, int32_t layer, int32_t which, int32_t pos0, int32_t n, float* host)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    return kv_copy(m, layer, which, pos0, n, host, true);
}

df_status df_write_kv(df_model* m, int32_t layer, int32_t which, int32_t pos0, int32_t n,
                      const float* host, int32_t kv_len_after)
{
    if (!m) return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    if (kv_len_after < 0 || kv_len_after > m->cfg.max_ctx)
        return set_err(m, DF_ERR_INVALID_ARGUMENT,
                       fmt("df_write_kv: kv_len_after %d outside [0, %d]", kv_len_after, m->cfg.max_ctx));
    df_status st = kv_copy(m, layer, which, pos0, n, const_cast<float*>(host), false);
    if (st == DF_OK) m->kv_len = kv_len_after;
    return st;
}

void* df_stream(const df_model* m)
{
    return m ? static_cast<void*>(m->stream) : nullptr;
}

df_status df_time_kernel(df_model* m, int32_t kernel, int32_t reps, double* mean_us)
{
    if (!m || !mean_us || reps <= 0 || kernel < 0 || kernel >= DF_K_COUNT)
        return DF_ERR_INVALID_ARGUMENT;
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    (void)hipSetDevice(m->device);
    Fail e{DF_OK, ""};
    m->pool.reset();
    StepBufs b{};
    if (!step_buffers(m, &b, &e)) return set_err(m, e.code, e.msg);
    float* lg = static_cast<float*>(m->pool.alloc(size_t(m->cfg.vocab) * 4, USAGE_DEVICE, &e));
    if (!lg) return set_err(m, e.code, e.msg);
    // The attention launch appends this step's K / V row at kv_len: on a full
    // cache that row is live, so the replay is refused rather than clamped.
    if (kernel == DF_K_ATTN && m->kv_len >= m->cfg.max_ctx)
        return set_err(m, DF_ERR_CONTEXT_FULL,
                       fmt("df_time_kernel: the cache is full (kv_len %d == max_ctx); the replay "
                           "would overwrite its last row", m->kv_len));
    const bool per_layer = kernel != DF_K_EMBED && kernel != DF_K_LOGITS && kernel != DF_K_ARGMAX;
    const int nl = per_layer ? m->cfg.n_layers : 1;
    if (nl == 0) return set_err(m, DF_ERR_INVALID_ARGUMENT, "df_time_kernel: no layers");
    // position of the replayed step: kv_len (the attention classes need a
    // free row there); the other classes only read it
    const int pos = m->kv_len < m->cfg.max_ctx ? m->kv_len : m->cfg.max_ctx - 1;
    const int splits = attn_splits(pos);
    hipError_t r = launch_set_state(m->state, pos, 0, 0, m->stream);
    if (r == hipSuccess) r = hipEventRecord(m->ev0, m->stream);
    for (int rep = 0; rep < reps && r == hipSuccess; ++rep)
        for (int l = 0; l < nl && r == hipSuccess; ++l)
            r = kernel == DF_K_ARGMAX
                    ? launch_argmax(lg, m->cfg.vocab, m->state, m->argmax_out, 0, nullptr, m->stream)
                : launch_class(m, b, kernel, l, splits, lg);
    if (r == hipSuccess) r = hipEventRecord(m->ev1, m->stream);
    if (r == hipSuccess) r = hipEventSynchronize(m->ev1);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, m->ev0, m->ev1);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("df_time_kernel: %s", hipGetErrorString(r)));
    }
    m->ev_kind = 0;
    *mean_us = double(ms) * 1e3 / double(reps * nl);
    return DF_OK;
}

df_status df_time_prefill(df_model* m, int32_t kernel, int32_t rows, int32_t reps, double* mean_us)
{
    if (!m || !mean_us || reps <= 0 || kernel < DF_K_PF_QKV || kernel > DF_K_PF_ROWS)
        return DF_ERR_INVALID_ARGUMENT;
    if (rows < 1 || rows > m->cfg.max_ctx - m->kv_len)
        return set_err(m, DF_ERR_INVALID_ARGUMENT,
                       fmt("df_time_prefill: rows = %d: expected 1..%d (max_ctx %d - kv_len %d: the "
                           "replay writes cache rows past kv_len only)",
                           rows, m->cfg.max_ctx - m->kv_len, m->cfg.max_ctx, m->kv_len));
    if (m->cfg.n_layers == 0) return set_err(m, DF_ERR_INVALID_ARGUMENT, "df_time_prefill: no layers");
    if (!bulk_supported(m))
        return set_err(m, DF_ERR_UNSUPPORTED_OP, "df_time_prefill: bulk prefill needs f16 or 8-bit weights");
    BusyGuard guard(m);
    if (!guard.ok) return DF_ERR_BUSY;
    (void)hipSetDevice(m->device);
    Fail e{DF_OK, ""};
    m->pool.reset();
    PfBufs b{};
    if (!pf_buffers(m, rows, &b, &e)) return set_err(m, e.code, e.msg);
    // Defined, non-constant inputs: pseudo-random activations. The matrix
    // cores draw more power on random operands than on zeros, and the
    // clocks follow, so zero inputs would time the GEMMs about 20% fast.
    const df_config& c = m->cfg;
    const size_t qd = size_t(c.n_heads) * c.head_dim, kvd = size_t(c.n_kv_heads) * c.head_dim;
    hipError_t r = launch_fill_random(b.x, int64_t(rows) * c.d_model, 0, 1u, m->stream);
    if (r == hipSuccess) r = launch_fill_random(b.h16, int64_t(rows) * c.d_model, 1, 2u, m->stream);
    if (r == hipSuccess) r = launch_fill_random(b.qkv, int64_t(rows) * int64_t(qd + 2 * kvd), 0, 3u, m->stream);
    if (r == hipSuccess) r = launch_fill_random(b.att16, int64_t(rows) * int64_t(qd), 1, 4u, m->stream);
    if (r == hipSuccess) r = launch_fill_random(b.mid16, int64_t(rows) * c.ffn_dim, 1, 5u, m->stream);
    const int nl = c.n_layers;
    // the attention reads q and the cache rows the row pass writes
    if (kernel == DF_K_PF_ATTN)
        for (int l = 0; l < nl && r == hipSuccess; ++l) r = pf_launch(m, b, DF_K_PF_ROWS, l, rows, m->kv_len);
    if (r == hipSuccess) r = hipEventRecord(m->ev0, m->stream);
    for (int rep = 0; rep < reps && r == hipSuccess; ++rep)
        for (int l = 0; l < nl && r == hipSuccess; ++l) r = pf_launch(m, b, kernel, l, rows, m->kv_len);
    if (r == hipSuccess) r = hipEventRecord(m->ev1, m->stream);
    if (r == hipSuccess) r = hipEventSynchronize(m->ev1);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, m->ev0, m->ev1);
    if (r != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, fmt("df_time_prefill: %s", hipGetErrorString(r)));
    }
    m->ev_kind = 0;
    *mean_us = double(ms) * 1e3 / double(reps * nl);
    return DF_OK;
}

df_status df_prefill_plan(const df_model* m, int32_t rows, int32_t* plan)
{
    if (!m || !plan || rows < 1) return DF_ERR_INVALID_ARGUMENT;
    const df_config& c = m->cfg;
    if (c.n_layers == 0 || !bulk_supported(m)) {
        for (int i = 0; i < 4; ++i) plan[i] = 0;
        return DF_OK;
    }
    const int64_t qd = int64_t(c.n_heads) * c.head_dim, kvd = int64_t(c.n_kv_heads) * c.head_dim;
    const bool q8 = m->layers[0].wqkv.scales != nullptr;
    // 8-bit weights from PF_DEQUANT_MIN_ROWS rows on: converted to f16 first
    // (pf_buffers / pf_launch), then the f16 GEMMs
    const bool first = q8 && rows >= PF_DEQUANT_MIN_ROWS;
    const bool in_gemm = q8 && !first;
    const bool gemma = c.arch == DF_ARCH_GEMMA3;
    const int64_t N[4] = {qd + 2 * kvd, c.d_model, c.ffn_dim, c.d_model};
    const int64_t K[4] = {c.d_model, qd, c.d_model, c.ffn_dim};
    const int mode[4] = {GEMM_STORE_F32, gemma ? GEMM_STORE_F32 : GEMM_ADD_F32, GEMM_SWIGLU_F16,
                         gemma ? GEMM_STORE_F32 : GEMM_ADD_F32};
    for (int i = 0; i < 4; ++i)
        plan[i] = gemm_plan(rows, N[i], K[i], i == 2 ? c.ffn_dim : 0, mode[i], in_gemm) |
                  (first ? GEMM_PLAN_DEQUANT_FIRST : 0);
    return DF_OK;
}

df_status df_profile(df_model* m, int32_t kernel, int32_t enable)
{
    if (!m || kernel < 0 || kernel >= DF_K_COUNT) return DF_ERR_INVALID_ARGUMENT;
    m->prof_kernel = enable ? kernel : -1;
    return DF_OK;
}

df_status df_profile_read(df_model* m, int32_t kernel, int64_t* launches, double* total_ms)
{
    if (!m || !launches || !total_ms || kernel < 0 || kernel >= DF_K_COUNT)
        return DF_ERR_INVALID_ARGUMENT;
    (void)hipSetDevice(m->device);
    if (hipStreamSynchronize(m->stream) != hipSuccess) {
        (void)hipGetLastError();
        return set_err(m, DF_ERR_DEVICE, "df_profile_read: synchronise failed");
    }
    double ms_sum = 0;
    for (size_t i = 0; i < m->prof_used; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, m->prof_events[i].first, m->prof_events[i].second) == hipSuccess)
            ms_sum += ms;
        else
            (void)hipGetLastError();
    }
    *launches = int64_t(m->prof_used);
    *total_ms = ms_sum;
    m->prof_used = 0;
    return DF_OK;
}

}  // extern "C"
