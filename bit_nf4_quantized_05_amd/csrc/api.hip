// extern "C" entry points of libqlora_nf4: argument checks, workspace layout and
// kernel sequencing. Every step of the layer runs in the kernels of quantize.hip,
// prologue.hip, gemm_nt.hip, gemv.hip, skinny.hip, lora_grads.hip and factors.hip; this file does
// no arithmetic on the data.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlora_nf4.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    g_err = std::string(where) + ": " + hipGetErrorString(e);
    return -4;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

constexpr int64_t kMaxBlocks = (int64_t{1} << 32) - 1;

bool nf4_counts(int64_t d_out, int64_t d_in, int64_t* n, int64_t* n_b, int64_t* n_g) {
    if (d_out < 1 || d_in < 1) return false;
    if (d_out > (int64_t{1} << 40) / d_in) return false;
    *n = d_out * d_in;
    *n_b = (*n + qn::kBlock - 1) / qn::kBlock;
    *n_g = (*n_b + qn::kGroup - 1) / qn::kGroup;
    return *n_b <= kMaxBlocks;
}

// The block-constant arrays of a quantised weight in format dq. Checks pointers and
// alignment; for QN_DQ_NONE, qconst and qmean are not part of the format (may be
// null) and readable stand-ins replace them, since kernels load them unconditionally.
int make_consts(int dq, const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                qn::BlockConsts* bc) {
    if (dq != QN_DQ_INT8 && dq != QN_DQ_FP8 && dq != QN_DQ_NONE) return fail(-1, "unknown second-level format");
    if (!codes || !qscale) return fail(-1, "null pointer argument");
    if (!aligned(qscale, 4)) return fail(-1, "misaligned pointer");
    if (dq == QN_DQ_NONE) {
        *bc = qn::BlockConsts{reinterpret_cast<const int8_t*>(codes), qscale, qscale, qn::kDqNone, 0};
        return 0;
    }
    if (!qconst || !qmean) return fail(-1, "null pointer argument");
    if (!aligned(qmean, 4)) return fail(-1, "misaligned pointer");
    *bc = qn::BlockConsts{qconst, qscale, qmean, dq == QN_DQ_FP8 ? qn::kDqFp8 : qn::kDqInt8, 8};
    return 0;
}

static_assert(QN_DQ_INT8 == qn::kDqInt8 && QN_DQ_FP8 == qn::kDqFp8 && QN_DQ_NONE == qn::kDqNone,
              "format codes");

struct QuantWs {
    int64_t absmax_off, limbs_off, bytes;
    int grid;
};

QuantWs quant_ws(int64_t n_b) {
    QuantWs w{};
    w.grid = qn::quant_grid(n_b);
    w.absmax_off = 0;
    w.limbs_off = align_up(n_b * 4, 256);
    w.bytes = w.limbs_off + align_up(static_cast<int64_t>(w.grid) * qn::kLimbs * 8, 256);
    return w;
}

struct LinWs {
    int64_t what, lora, adapt, adapt2, t, part, gpart, ppart, bytes;
    int r_pad;
};

// fp32 partials of a K-split LoRA pre-pass over M tokens and K columns (0 if unsplit)
int64_t prepass_part_bytes(int64_t M, int64_t K, int r) {
    const qn::PrepassSplit ps = qn::prepass_split(M, K);
    return ps.splits > 1 ? 4 * static_cast<int64_t>(ps.splits) * M * 32 * ((r + 31) / 32) : 0;
}

// Workspace layout of one linear call. The forward with d_seq <= kSkinnyMaxTokens streams
// the packed codes (GEMV or small batch) and needs only its partial sums; every other
// call dequantises W into the workspace and runs the GEMM. Regions a call does not use
// have size 0.
LinWs linear_ws(int64_t d_out, int64_t d_in, int64_t d_seq, int r, bool bwd) {
    LinWs w{};
    w.r_pad = static_cast<int>(align_up(r, 64));
    const bool streams = !bwd && d_seq <= qn::kSkinnyMaxTokens;
    const bool gemm = !streams;
    int64_t off = 0;
    w.what = off;   if (gemm) off += align_up(2 * d_out * d_in, 256);                        // W_hat or W_hat^T
    w.lora = off;   if (gemm) off += align_up(2 * d_seq * w.r_pad, 256);                     // s(XA^T) or s(dY B)
    w.adapt = off;  if (gemm) off += align_up(2 * (bwd ? d_in : d_out) * w.r_pad, 256);      // B padded or A^T padded
    w.adapt2 = off;                                                                          // B^T (unless the pre-pass reads B)
    if (bwd && !qn::prepass_takes_kmajor(r)) off += align_up(2 * static_cast<int64_t>(r) * d_out, 256);
    w.t = off;                                                                               // GEMV: partial A x
    if (streams && qn::gemv_takes_tokens(d_seq, d_out, d_in, r)) off += align_up(4 * qn::gemv_part_floats(d_seq, d_in, r), 256);
    w.part = off;                                                                            // small batch: K-split partials
    if (streams && !qn::gemv_takes_tokens(d_seq, d_out, d_in, r))
        off += align_up(4 * static_cast<int64_t>(qn::skinny_splits(d_in, d_seq)) * d_seq * (d_out + w.r_pad), 256);
    w.gpart = off;                                                                           // GEMM K-split partials (few tiles)
    if (gemm) off += align_up(4 * (bwd ? qn::gemm_split_part_floats(d_seq, d_in, d_out)
                                       : qn::gemm_split_part_floats(d_seq, d_out, d_in)), 256);
    w.ppart = off;                                                                           // pre-pass K-split partials
    if (gemm) off += align_up(bwd ? prepass_part_bytes(d_seq, d_out, r) : prepass_part_bytes(d_seq, d_in, r), 256);
    w.bytes = off;
    return w;
}

bool linear_sizes_ok(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    return d_out >= 1 && d_in >= 1 && d_seq >= 1 && r >= 1 && r <= 256 && d_out <= (int64_t{1} << 40) / d_in &&
           d_seq <= INT32_MAX;
}

// Checks of a linear call; `in` [d_seq, in_cols] with row stride ldi, `out` [d_seq, out_cols]
// with row stride ldo (in elements).
int check_linear(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean, int dq,
                 int64_t d_out, int64_t d_in, const uint16_t* A, const uint16_t* B, int r,
                 const uint16_t* in, int64_t ldi, int64_t d_seq, uint16_t* out, int64_t ldo, bool bwd, void* ws,
                 int64_t ws_bytes, LinWs* lw, qn::BlockConsts* bc) {
    if (int rc = make_consts(dq, codes, qconst, qscale, qmean, bc)) return rc;
    if (!A || !B || !in || !out || !ws) return fail(-1, "null pointer argument");
    if (d_out < 1 || d_in < 1 || d_seq < 1) return fail(-1, "sizes must be >= 1");
    if (r < 1 || r > 256) return fail(-1, "r must be in [1, 256]");
    const int64_t in_cols = bwd ? d_out : d_in, out_cols = bwd ? d_in : d_out;
    if (ldi < in_cols || ldo < out_cols) return fail(-1, "a leading dimension is smaller than its row");
    if (ldi % 8 != 0 || ldo % 8 != 0) return fail(-1, "leading dimensions must be multiples of 8 elements");
    if (!aligned(codes, 16) || !aligned(A, 16) || !aligned(B, 16) || !aligned(in, 16) ||
        !aligned(out, 16) || !aligned(ws, 256))
        return fail(-1, "misaligned pointer (16 B for arrays, 256 B for the workspace)");
    if (d_in % 64 != 0 || d_out % 64 != 0) return fail(-2, "d_in and d_out must be multiples of 64");
    if (d_in > INT32_MAX || d_out > INT32_MAX || d_seq > INT32_MAX) return fail(-2, "dimension too large");
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return fail(-2, "weight too large");
    // the GEMM addresses each operand with 32-bit byte offsets
    const int64_t kMaxBytes = int64_t{1} << 32;
    if (2 * n >= kMaxBytes || 2 * d_seq * std::max(ldi, ldo) >= kMaxBytes)
        return fail(-2, "an operand reaches 4 GiB");
    *lw = linear_ws(d_out, d_in, d_seq, r, bwd);
    if (ws_bytes < lw->bytes) return fail(-3, "workspace too small");
    return 0;
}

}  // namespace

// ---- optional kernel timing -------------------------------------------------
namespace qn {
namespace {
struct ProfRec {
    const char* name;
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof;
// Events are created once and reused: creating one per launch costs the host more than
// a short kernel runs, which left the device idle between launches while timing was on.
std::vector<hipEvent_t> g_pool;
constexpr size_t kPoolPrefill = 1024;

hipEvent_t take_event_locked() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

void prof_clear_locked() {
    for (auto& r : g_prof) {
        g_pool.push_back(r.start);
        g_pool.push_back(r.stop);
    }
    g_prof.clear();
}
}  // namespace

void* prof_begin(hipStream_t st) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return nullptr;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t e = take_event_locked();
    if (!e) return nullptr;
    if (hipEventRecord(e, st) != hipSuccess) {
        g_pool.push_back(e);
        return nullptr;
    }
    return e;
}

void prof_end(void* token, const char* name, hipStream_t st) {
    if (!token) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t e = take_event_locked();
    if (!e || hipEventRecord(e, st) != hipSuccess) {
        g_pool.push_back(static_cast<hipEvent_t>(token));
        if (e) g_pool.push_back(e);
        return;
    }
    g_prof.push_back({name, static_cast<hipEvent_t>(token), e});
}
}  // namespace qn

namespace {

// The forward once the arguments are checked: d_seq == 1 (and up to 3 tokens when r <= 16
// and d_in <= 4096) streams the codes (GEMV), d_seq <= 64 runs the small-batch kernel,
// otherwise dequantise + pre-pass + GEMM.
// forward GEMM form for d_seq > 64 (qlora_set_fwd_gemm)
std::atomic<int> g_fwd_gemm{QN_FWD_GEMM_AUTO};

// AUTO picks the in-GEMM dequantisation for a weight whose bf16 copy would not fit the
// 256 MB Infinity Cache (d_out d_in >= 2^27) at up to 1024 tokens (at most 4 tile rows of
// 256 tokens, each of which dequantises every weight again); otherwise W_hat is staged.
// Measured at 65..2048 tokens: fused / staged call time 0.55..0.95 for 28672 x 8192 up
// to 1024 tokens and 1.10 at 2048; 0.98..1.37 for the 11008 x 4096 and 4096 x 11008 MLP
// layers and 1.00..1.23 for 4096 x 4096, whose staged W_hat stays in the cache.
bool fwd_gemm_fused(int64_t d_seq, int64_t d_out, int64_t d_in) {
    const int form = g_fwd_gemm.load(std::memory_order_relaxed);
    if (form != QN_FWD_GEMM_AUTO) return form == QN_FWD_GEMM_FUSED;
    return d_out * d_in >= (int64_t{1} << 27) && d_seq <= 1024;
}

int linear_fwd_run(const uint8_t* codes, const qn::BlockConsts& bc, int64_t d_out, int64_t d_in,
                   const uint16_t* A, const uint16_t* B, int r, float s, const uint16_t* X, int64_t ldx,
                   int64_t d_seq, uint16_t* Y, int64_t ldy, char* ws, const LinWs& lw, hipStream_t st) {
    hipError_t e;
    if (qn::gemv_takes_tokens(d_seq, d_out, d_in, r)) {
        e = qn::launch_gemv_nf4(codes, bc, d_out, d_in, A, B, r, s, X, ldx, d_seq, Y, ldy,
                                reinterpret_cast<float*>(ws + lw.t), st);
        if (e != hipSuccess) return hip_fail(e, "qlora_linear_fwd (gemv)");
        return 0;
    }
    if (d_seq <= qn::kSkinnyMaxTokens) {
        // few tokens: the codes streamed once, A x in the same launch
        float* part = reinterpret_cast<float*>(ws + lw.part);
        float* part_a = part + static_cast<int64_t>(qn::skinny_splits(d_in, d_seq)) * d_seq * d_out;
        if ((e = qn::launch_skinny_nf4(codes, bc, d_out, d_in, X, ldx, d_seq, A, B, r, lw.r_pad, s,
                                       part, part_a, Y, ldy, st)) != hipSuccess)
            return hip_fail(e, "qlora_linear_fwd (small batch)");
        return 0;
    }
    const bool fused = fwd_gemm_fused(d_seq, d_out, d_in);
    uint16_t* what = fused ? nullptr : reinterpret_cast<uint16_t*>(ws + lw.what);
    uint16_t* t = reinterpret_cast<uint16_t*>(ws + lw.lora);
    uint16_t* bpad = reinterpret_cast<uint16_t*>(ws + lw.adapt);
    const bool pad = r != lw.r_pad;
    // T = s (X A^T) + B padded to r_pad columns (+ the dequantised W_hat when staged), in
    // one launch
    if ((e = qn::launch_prologue(codes, bc, d_out, d_in, false, what, X, ldx, d_seq, d_in,
                                 A, d_in, false, r, s, t, lw.r_pad, pad ? 1 : 0, B, bpad, d_out, r,
                                 reinterpret_cast<float*>(ws + lw.ppart), st)) != hipSuccess)
        return hip_fail(e, "qlora_linear_fwd (prologue)");
    if ((e = qn::launch_gemm_nt(X, ldx, what, d_in, d_in, t, lw.r_pad, pad ? bpad : B, lw.r_pad, lw.r_pad, Y,
                                ldy, d_seq, d_out, reinterpret_cast<float*>(ws + lw.gpart), st,
                                fused ? codes : nullptr, &bc)) != hipSuccess)
        return hip_fail(e, "qlora_linear_fwd (gemm)");
    return 0;
}

}  // namespace

// workspace of qlora_lora_grads
namespace {
struct GradWs {
    int64_t tp, up, bt, part, ppart, ppart1, bytes;
    int r_pad;
};

GradWs grad_ws(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    GradWs w{};
    w.r_pad = static_cast<int>(align_up(r, 64));
    int64_t off = 0;
    w.tp = off;   off += align_up(2 * d_seq * w.r_pad, 256);                        // T' = bf16(s X A^T)
    w.up = off;   off += align_up(2 * d_seq * w.r_pad, 256);                        // U' = bf16(s dY B)
    w.bt = off;   off += align_up(2 * static_cast<int64_t>(r) * d_out, 256);        // B^T (unless the pre-pass reads B)
    w.part = off; off += align_up(4 * qn::lora_grads_partials(d_out, d_in, d_seq, r), 256);
    w.ppart = off; off += align_up(prepass_part_bytes(d_seq, d_in, r), 256);       // X A^T K-split partials
    w.ppart1 = off; off += align_up(prepass_part_bytes(d_seq, d_out, r), 256);     // dY B K-split partials
    w.bytes = off;
    return w;
}
}  // namespace

namespace qn {
// polls a persistent one-token GEMV workgroup makes for each published A x slice word
// before forming every slice itself (process-wide, gemv.hip); returns the previous value
int set_ax_polls(int polls);
}  // namespace qn

// ---- scratch of the allocation-free forward ---------------------------------
// One static device array (each device holds its own copy, from module load until the
// process ends). Host code never uses the array's name as an address: the address of
// each device's copy is taken once with hipGetSymbolAddress, with that device current,
// and kept per device.
namespace {
constexpr int64_t kNoAllocScratchBytes = QN_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (nullptr and the error text set on failure).
char* scratch_of_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        hip_fail(e, "hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        fail(-4, "device index out of range");
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
            return nullptr;
        }
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int qn_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(qn::g_prof_mu);
    qn::prof_clear_locked();
    while (on && qn::g_pool.size() < qn::kPoolPrefill) {
        hipEvent_t e = nullptr;
        const hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return hip_fail(err, "qn_profile_enable");
        qn::g_pool.push_back(e);
    }
    qn::g_prof_on.store(on != 0);
    return 0;
}

int qn_profile_read(char* names, int name_len, int64_t* launches, double* total_ms, int cap) {
    if (!names || !launches || !total_ms || name_len < 2 || cap < 0) return fail(-1, "bad argument");
    std::lock_guard<std::mutex> lk(qn::g_prof_mu);
    std::map<std::string, std::pair<int64_t, double>> agg;
    for (auto& r : qn::g_prof) {
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "qn_profile_read");
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "qn_profile_read");
        auto& a = agg[r.name];
        a.first += 1;
        a.second += ms;
    }
    int i = 0;
    for (auto& kv : agg) {
        if (i >= cap) break;
        std::strncpy(names + static_cast<size_t>(i) * name_len, kv.first.c_str(), name_len - 1);
        names[static_cast<size_t>(i) * name_len + name_len - 1] = 0;
        launches[i] = kv.second.first;
        total_ms[i] = kv.second.second;
        ++i;
    }
    return static_cast<int>(agg.size());
}

int qn_profile_durations(const char* name, float* ms, int cap) {
    if (!name || (!ms && cap > 0) || cap < 0) return fail(-1, "bad argument");
    std::lock_guard<std::mutex> lk(qn::g_prof_mu);
    int n = 0;
    for (auto& r : qn::g_prof) {
        if (std::strcmp(r.name, name) != 0) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "qn_profile_durations");
        float t = 0.0f;
        e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "qn_profile_durations");
        if (n < cap) ms[n] = t;
        ++n;
    }
    return n;
}

int qn_version(void) { return 100; }

const char* qn_last_error(void) { return g_err.c_str(); }

int qn_codebook(float* out16) {
    if (!out16) return fail(-1, "null pointer argument");
    std::memcpy(out16, qn::tables().code, sizeof(float) * 16);
    return 0;
}

int qn_nf4_sizes(int64_t d_out, int64_t d_in, int64_t* codes_bytes, int64_t* n_blocks, int64_t* n_groups) {
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return fail(-1, "bad weight shape");
    if (codes_bytes) *codes_bytes = n_b * (qn::kBlock / 2);
    if (n_blocks) *n_blocks = n_b;
    if (n_groups) *n_groups = n_g;
    return 0;
}

int qn_nf4_sizes_ex(int64_t d_out, int64_t d_in, int dq, int64_t* codes_bytes, int64_t* qconst_entries,
                    int64_t* qscale_entries) {
    if (dq != QN_DQ_INT8 && dq != QN_DQ_FP8 && dq != QN_DQ_NONE) return fail(-1, "unknown second-level format");
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return fail(-1, "bad weight shape");
    if (codes_bytes) *codes_bytes = n_b * (qn::kBlock / 2);
    if (qconst_entries) *qconst_entries = dq == QN_DQ_NONE ? 0 : n_b;
    if (qscale_entries) *qscale_entries = dq == QN_DQ_NONE ? n_b : n_g;
    return 0;
}

int64_t nf4_quantize_workspace_bytes(int64_t d_out, int64_t d_in) {
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return 0;
    return quant_ws(n_b).bytes;
}

int nf4_quantize_ex(const float* W, int64_t d_out, int64_t d_in, int dq, uint8_t* codes, int8_t* qconst,
                    float* qscale, float* qmean, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!W || !workspace) return fail(-1, "null pointer argument");
    qn::BlockConsts bc;
    if (int rc = make_consts(dq, codes, qconst, qscale, qmean, &bc)) return rc;
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return fail(-1, "bad weight shape");
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(workspace, 256)) return fail(-1, "misaligned pointer");
    const QuantWs w = quant_ws(n_b);
    if (workspace_bytes < w.bytes) return fail(-3, "workspace too small");
    char* ws = static_cast<char*>(workspace);
    hipError_t e = qn::launch_quantize(W, n, n_b, n_g, bc.fmt, codes, qconst, qscale, qmean,
                                       reinterpret_cast<float*>(ws + w.absmax_off),
                                       reinterpret_cast<unsigned long long*>(ws + w.limbs_off), w.grid,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "nf4_quantize");
    return 0;
}

int nf4_quantize(const float* W, int64_t d_out, int64_t d_in, uint8_t* codes, int8_t* qconst,
                 float* qscale, float* qmean, void* workspace, int64_t workspace_bytes, void* stream) {
    return nf4_quantize_ex(W, d_out, d_in, QN_DQ_INT8, codes, qconst, qscale, qmean, workspace, workspace_bytes,
                           stream);
}

int nf4_double_dequant_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                          int64_t d_out, int64_t d_in, int dq, uint16_t* W_bf16, void* stream) {
    qn::BlockConsts bc;
    if (int rc = make_consts(dq, codes, qconst, qscale, qmean, &bc)) return rc;
    if (!W_bf16) return fail(-1, "null pointer argument");
    int64_t n, n_b, n_g;
    if (!nf4_counts(d_out, d_in, &n, &n_b, &n_g)) return fail(-1, "bad weight shape");
    if (!aligned(codes, 16) || !aligned(W_bf16, 16)) return fail(-1, "misaligned pointer");
    hipError_t e = qn::launch_dequant_rows(codes, bc, n, W_bf16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "nf4_double_dequant");
    return 0;
}

int nf4_double_dequant(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                       int64_t d_out, int64_t d_in, uint16_t* W_bf16, void* stream) {
    return nf4_double_dequant_ex(codes, qconst, qscale, qmean, d_out, d_in, QN_DQ_INT8, W_bf16, stream);
}

int64_t qlora_linear_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    if (!linear_sizes_ok(d_out, d_in, d_seq, r)) return 0;
    return std::max(linear_ws(d_out, d_in, d_seq, r, false).bytes, linear_ws(d_out, d_in, d_seq, r, true).bytes);
}

int64_t qlora_linear_fwd_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    if (!linear_sizes_ok(d_out, d_in, d_seq, r)) return 0;
    return linear_ws(d_out, d_in, d_seq, r, false).bytes;
}

int64_t qlora_linear_bwd_x_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    if (!linear_sizes_ok(d_out, d_in, d_seq, r)) return 0;
    return linear_ws(d_out, d_in, d_seq, r, true).bytes;
}

int qlora_linear_fwd_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                        int64_t d_out, int64_t d_in, int dq, const uint16_t* A, const uint16_t* B, int r, float s,
                        const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy, void* workspace,
                        int64_t workspace_bytes, void* stream) {
    LinWs lw;
    qn::BlockConsts bc;
    int rc = check_linear(codes, qconst, qscale, qmean, dq, d_out, d_in, A, B, r, X, ldx, d_seq, Y, ldy, false,
                          workspace, workspace_bytes, &lw, &bc);
    if (rc) return rc;
    return linear_fwd_run(codes, bc, d_out, d_in, A, B, r, s, X, ldx, d_seq, Y, ldy, static_cast<char*>(workspace),
                          lw, static_cast<hipStream_t>(stream));
}

int qlora_set_ax_wait(int polls) {
    if (polls < 0) return -1;
    return qn::set_ax_polls(polls);
}

int qlora_set_fwd_gemm(int form) {
    if (form != QN_FWD_GEMM_AUTO && form != QN_FWD_GEMM_STAGED && form != QN_FWD_GEMM_FUSED) return -1;
    return g_fwd_gemm.exchange(form);
}

int qlora_linear_fwd(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                     int64_t d_out, int64_t d_in, const uint16_t* A, const uint16_t* B, int r, float s,
                     const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy, void* workspace,
                     int64_t workspace_bytes, void* stream) {
    return qlora_linear_fwd_ex(codes, qconst, qscale, qmean, d_out, d_in, QN_DQ_INT8, A, B, r, s, X, ldx, d_seq, Y,
                               ldy, workspace, workspace_bytes, stream);
}

int qlora_linear_fwd_noalloc(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                             int64_t d_out, int64_t d_in, int dq, const uint16_t* A, const uint16_t* B, int r,
                             float s, const uint16_t* X, int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy,
                             void* stream) {
    if (d_seq < 1) return fail(-1, "sizes must be >= 1");
    if (d_seq > qn::kSkinnyMaxTokens)
        return fail(-2, "qlora_linear_fwd_noalloc takes at most 64 tokens (more would dequantise W into scratch)");
    char* ws = scratch_of_current_device();
    if (ws == nullptr) return -4;
    LinWs lw;
    qn::BlockConsts bc;
    int rc = check_linear(codes, qconst, qscale, qmean, dq, d_out, d_in, A, B, r, X, ldx, d_seq, Y, ldy, false, ws,
                          kNoAllocScratchBytes, &lw, &bc);
    if (rc == -3) return fail(-2, "qlora_linear_fwd_noalloc: these sizes need more than the static scratch holds");
    if (rc) return rc;
    return linear_fwd_run(codes, bc, d_out, d_in, A, B, r, s, X, ldx, d_seq, Y, ldy, ws, lw,
                          static_cast<hipStream_t>(stream));
}

int qlora_linear_bwd_x_ex(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                          int64_t d_out, int64_t d_in, int dq, const uint16_t* A, const uint16_t* B, int r,
                          float s, const uint16_t* dY, int64_t lddy, int64_t d_seq, uint16_t* dX, int64_t lddx,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    LinWs lw;
    qn::BlockConsts bc;
    int rc = check_linear(codes, qconst, qscale, qmean, dq, d_out, d_in, A, B, r, dY, lddy, d_seq, dX, lddx, true,
                          workspace, workspace_bytes, &lw, &bc);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    uint16_t* whatT = reinterpret_cast<uint16_t*>(ws + lw.what);
    uint16_t* u = reinterpret_cast<uint16_t*>(ws + lw.lora);
    uint16_t* atpad = reinterpret_cast<uint16_t*>(ws + lw.adapt);
    uint16_t* bt = reinterpret_cast<uint16_t*>(ws + lw.adapt2);
    hipError_t e;
    // the pre-pass reads B itself (k-major) where it can; else K-contiguous rows of B^T
    const bool km = qn::prepass_takes_kmajor(r);
    if (!km && (e = qn::launch_transpose_pad(B, d_out, r, bt, d_out, st)) != hipSuccess)
        return hip_fail(e, "qlora_linear_bwd_x (B^T)");
    // dequant W_hat^T + U = s (dY B) + A^T padded to r_pad columns, in one launch
    if ((e = qn::launch_prologue(codes, bc, d_out, d_in, true, whatT, dY, lddy, d_seq, d_out,
                                 km ? B : bt, d_out, km, r, s, u, lw.r_pad, 2, A, atpad, r, d_in,
                                 reinterpret_cast<float*>(ws + lw.ppart), st)) != hipSuccess)
        return hip_fail(e, "qlora_linear_bwd_x (prologue)");
    if ((e = qn::launch_gemm_nt(dY, lddy, whatT, d_out, d_out, u, lw.r_pad, atpad, lw.r_pad, lw.r_pad, dX,
                                lddx, d_seq, d_in, reinterpret_cast<float*>(ws + lw.gpart), st)) != hipSuccess)
        return hip_fail(e, "qlora_linear_bwd_x (gemm)");
    return 0;
}

int qlora_linear_bwd_x(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                       int64_t d_out, int64_t d_in, const uint16_t* A, const uint16_t* B, int r, float s,
                       const uint16_t* dY, int64_t lddy, int64_t d_seq, uint16_t* dX, int64_t lddx, void* workspace,
                       int64_t workspace_bytes, void* stream) {
    return qlora_linear_bwd_x_ex(codes, qconst, qscale, qmean, d_out, d_in, QN_DQ_INT8, A, B, r, s, dY, lddy, d_seq,
                                 dX, lddx, workspace, workspace_bytes, stream);
}

// ---- quantised low-rank factors (W ~ Q + L R) --------------------------------
int int8_quantize(const float* W, int64_t rows, int64_t cols, int8_t* q, float* absmax, void* stream) {
    if (!W || !q || !absmax) return fail(-1, "null pointer argument");
    int64_t n, n_b, n_g;
    if (!nf4_counts(rows, cols, &n, &n_b, &n_g)) return fail(-1, "bad shape");
    if (!aligned(W, 16) || !aligned(q, 16) || !aligned(absmax, 4)) return fail(-1, "misaligned pointer");
    hipError_t e = qn::launch_int8_quantize(W, n, q, absmax, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "int8_quantize");
    return 0;
}

int int8_dequant(const int8_t* q, const float* absmax, int64_t rows, int64_t cols, uint16_t* W_bf16, void* stream) {
    if (!q || !absmax || !W_bf16) return fail(-1, "null pointer argument");
    int64_t n, n_b, n_g;
    if (!nf4_counts(rows, cols, &n, &n_b, &n_g)) return fail(-1, "bad shape");
    if (!aligned(q, 16) || !aligned(absmax, 4) || !aligned(W_bf16, 16)) return fail(-1, "misaligned pointer");
    hipError_t e = qn::launch_int8_dequant(q, absmax, n, W_bf16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "int8_dequant");
    return 0;
}

int64_t qlr_linear_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    if (!linear_sizes_ok(d_out, d_in, d_seq, r)) return 0;
    return linear_ws(d_out, d_in, d_seq, r, false).bytes + align_up(2 * r * d_in, 256) + align_up(2 * d_out * r, 256);
}

int qlr_linear_fwd(const uint8_t* codes, const int8_t* qconst, const float* qscale, const float* qmean,
                   int64_t d_out, int64_t d_in, int dq, int a_bits, const void* a_codes, const float* a_scale,
                   int b_bits, const void* b_codes, const float* b_scale, int r, float s, const uint16_t* X,
                   int64_t ldx, int64_t d_seq, uint16_t* Y, int64_t ldy, void* workspace, int64_t workspace_bytes,
                   void* stream) {
    if ((a_bits != 4 && a_bits != 8) || (b_bits != 4 && b_bits != 8)) return fail(-1, "factor bits must be 4 or 8");
    if (!a_codes || !a_scale || !b_codes || !b_scale) return fail(-1, "null pointer argument");
    if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4))
        return fail(-1, "misaligned pointer");
    if (!linear_sizes_ok(d_out, d_in, d_seq, r)) return fail(-1, "sizes must be >= 1, r <= 256");
    // the dequantised factors sit after the forward's workspace (A [r, d_in], then B [d_out, r])
    const LinWs lw0 = linear_ws(d_out, d_in, d_seq, r, false);
    if (workspace_bytes < qlr_linear_workspace_bytes(d_out, d_in, d_seq, r)) return fail(-3, "workspace too small");
    char* ws = static_cast<char*>(workspace);
    uint16_t* a_hat = reinterpret_cast<uint16_t*>(ws + lw0.bytes);
    uint16_t* b_hat = reinterpret_cast<uint16_t*>(ws + lw0.bytes + align_up(2 * r * d_in, 256));
    LinWs lw;
    qn::BlockConsts bc;
    int rc = check_linear(codes, qconst, qscale, qmean, dq, d_out, d_in, a_hat, b_hat, r, X, ldx, d_seq, Y, ldy,
                          false, workspace, workspace_bytes, &lw, &bc);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    struct { int bits; const void* codes; const float* scale; int64_t n; uint16_t* out; } f[2] = {
        {a_bits, a_codes, a_scale, static_cast<int64_t>(r) * d_in, a_hat},
        {b_bits, b_codes, b_scale, d_out * static_cast<int64_t>(r), b_hat}};
    for (auto& fa : f) {
        if (fa.bits == 4) {
            const uint8_t* c = static_cast<const uint8_t*>(fa.codes);
            e = qn::launch_dequant_rows(c, qn::BlockConsts{reinterpret_cast<const int8_t*>(c), fa.scale, fa.scale,
                                                           qn::kDqNone, 0},
                                        fa.n, fa.out, st);
        } else {
            e = qn::launch_int8_dequant(static_cast<const int8_t*>(fa.codes), fa.scale, fa.n, fa.out, st);
        }
        if (e != hipSuccess) return hip_fail(e, "qlr_linear_fwd (factors)");
    }
    return linear_fwd_run(codes, bc, d_out, d_in, a_hat, b_hat, r, s, X, ldx, d_seq, Y, ldy, ws, lw, st);
}

// ---- adapter gradients ----------------------------------------------------

int64_t qlora_lora_grads_workspace_bytes(int64_t d_out, int64_t d_in, int64_t d_seq, int r) {
    if (d_out < 1 || d_in < 1 || d_seq < 1 || r < 1 || r > 256) return 0;
    return grad_ws(d_out, d_in, d_seq, r).bytes;
}

int qlora_lora_grads(const uint16_t* A, const uint16_t* B, int r, float s, const uint16_t* X, int64_t ldx,
                     const uint16_t* dY, int64_t lddy, int64_t d_out, int64_t d_in, int64_t d_seq, float* dA,
                     float* dB, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!A || !B || !X || !dY || !dA || !dB || !workspace) return fail(-1, "null pointer argument");
    if (d_out < 1 || d_in < 1 || d_seq < 1) return fail(-1, "sizes must be >= 1");
    if (r < 1 || r > 256) return fail(-1, "r must be in [1, 256]");
    if (ldx < d_in || lddy < d_out) return fail(-1, "a leading dimension is smaller than its row");
    if (ldx % 8 != 0 || lddy % 8 != 0) return fail(-1, "leading dimensions must be multiples of 8 elements");
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(X, 16) || !aligned(dY, 16) || !aligned(dA, 16) ||
        !aligned(dB, 16) || !aligned(workspace, 256))
        return fail(-1, "misaligned pointer (16 B for arrays, 256 B for the workspace)");
    if (d_in % 64 != 0 || d_out % 64 != 0) return fail(-2, "d_in and d_out must be multiples of 64");
    if (d_in > INT32_MAX || d_out > INT32_MAX || d_seq > INT32_MAX) return fail(-2, "dimension too large");
    if (2 * d_seq * std::max(ldx, lddy) >= (int64_t{1} << 32)) return fail(-2, "an operand reaches 4 GiB");
    const GradWs gw = grad_ws(d_out, d_in, d_seq, r);
    if (workspace_bytes < gw.bytes) return fail(-3, "workspace too small");
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    uint16_t* tp = reinterpret_cast<uint16_t*>(ws + gw.tp);
    uint16_t* up = reinterpret_cast<uint16_t*>(ws + gw.up);
    uint16_t* bt = reinterpret_cast<uint16_t*>(ws + gw.bt);
    float* part = reinterpret_cast<float*>(ws + gw.part);
    hipError_t e;
    // T' = bf16(s X A^T) and U' = bf16(s dY B): the forward's and the input gradient's
    // pre-passes (without the dequantisation) in one launch; U' on B itself where it can
    const bool km = qn::prepass_takes_kmajor(r);
    if (!km && (e = qn::launch_transpose_pad(B, d_out, r, bt, d_out, st)) != hipSuccess)
        return hip_fail(e, "qlora_lora_grads (B^T)");
    if ((e = qn::launch_prepass_pair(X, ldx, d_in, A, d_in, tp, reinterpret_cast<float*>(ws + gw.ppart),
                                     dY, lddy, d_out, km ? B : bt, d_out, km, up,
                                     reinterpret_cast<float*>(ws + gw.ppart1), d_seq, r, s, gw.r_pad, st)) !=
        hipSuccess)
        return hip_fail(e, "qlora_lora_grads (X A^T, dY B)");
    if ((e = qn::launch_lora_grads(X, ldx, dY, lddy, tp, up, d_out, d_in, d_seq, r, gw.r_pad, part, dA, dB, st)) !=
        hipSuccess)
        return hip_fail(e, "qlora_lora_grads (reduction)");
    return 0;
}

}  // extern "C"
