// libkvq C ABI: argument validation, block planning and launch sequencing.
// The operations themselves are defined in include/kvq.h; every step runs in
// the HIP kernels of kvq_eval.hip, kvq_solve.hip and kvq_quant.hip.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "kvq_internal.h"

// Device scratch of kvq_admit_noalloc: the solve's workspace (header and
// scan tile sums), then the one-launch admission's published words, for
// callers that cannot allocate.  Each device holds its
// own copy for the life of the process; host code reaches it only through
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kvq::kNoAllocScratchBytes];

namespace kvq {

void* staging_buffer(void** dev) {
    // One pinned buffer per host thread: a copy into pageable memory costs a
    // staged transfer (about 10 us more per call on MI355X).  It is never
    // freed, so no HIP call runs while the process shuts down.
    thread_local void* buf = nullptr;
    thread_local void* dbuf = nullptr;
    thread_local bool tried = false;
    if (!tried) {
        tried = true;
        if (hipHostMalloc(&buf, kStagingBytes, hipHostMallocDefault) != hipSuccess) buf = nullptr;
        if (buf && hipHostGetDevicePointer(&dbuf, buf, 0) != hipSuccess) dbuf = nullptr;
    }
    if (dev) *dev = dbuf;
    return buf;
}

hipError_t read_back(void* dst, const void* src, size_t bytes, hipStream_t st, bool staging) {
    void* buf = staging ? staging_buffer(nullptr) : nullptr;
    if (!buf || bytes > kStagingBytes) {
        const hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, st);
        return e == hipSuccess ? hipStreamSynchronize(st) : e;
    }
    hipError_t e = hipMemcpyAsync(buf, src, bytes, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess) memcpy(dst, buf, bytes);
    return e;
}

}  // namespace kvq

namespace {

thread_local std::string g_err;

kvq_status fail(kvq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

kvq_status ok() {
    g_err.clear();
    return KVQ_OK;
}

kvq_status hip_fail(hipError_t e, const char* where) {
    return fail(KVQ_EHIP, "%s: %s", where, hipGetErrorString(e));
}

int distinct_quantile_ranks(int n, int s, int32_t* out) {
    // sorted distinct ranks j (n-1)/(k-1) rounded half up over k = 2..s
    int32_t all[(KVQ_MAX_S + 1) * KVQ_MAX_S];
    int cnt = 0;
    for (int k = 2; k <= s; ++k)
        for (int j = 0; j < k; ++j) all[cnt++] = kvq::quantile_rank(j, k, n);
    for (int a = 1; a < cnt; ++a)  // insertion sort (at most 135 values)
        for (int b = a; b > 0 && all[b - 1] > all[b]; --b) {
            const int32_t tmp = all[b];
            all[b] = all[b - 1];
            all[b - 1] = tmp;
        }
    int u = 0;
    for (int a = 0; a < cnt; ++a)
        if (u == 0 || all[a] != all[u - 1]) all[u++] = all[a];
    if (out)
        for (int a = 0; a < u && a < kvq::kMaxStats; ++a) out[a] = all[a];
    return u;
}

void build_rank_table(const kvq_plan& p, kvq::RankTable& rt) {
    memset(&rt, 0, sizeof rt);
    if (p.search != KVQ_GRIDS) return;
    rt.n_stats = distinct_quantile_ranks(p.d_block, p.s, rt.rank);
    for (int k = 2; k <= p.s; ++k)
        for (int j = 0; j < k; ++j) {
            const int q = kvq::quantile_rank(j, k, p.d_block);
            for (int c = 0; c < rt.n_stats; ++c)
                if (rt.rank[c] == q) rt.col[k][j] = (uint8_t)c;
        }
}

// The rank table of a plan, rebuilt only when the block size, s or the
// search differ from the calling thread's previous call.
void rank_table(const kvq_plan& p, kvq::RankTable& rt) {
    thread_local int key_n = -1, key_s = -1, key_search = -1;
    thread_local kvq::RankTable cached;
    if (p.d_block != key_n || p.s != key_s || p.search != key_search) {
        build_rank_table(p, cached);
        key_n = p.d_block;
        key_s = p.s;
        key_search = p.search;
    }
    rt = cached;
}

bool valid_plan(const kvq_plan* p) {
    return p && p->n_blocks >= 0 && p->d_block >= 2 && p->d_block <= KVQ_MAX_BLOCK && p->s >= 2 &&
           p->s <= KVQ_MAX_S &&
           (p->search == KVQ_GRIDS || p->search == KVQ_EXACT_DP || p->search == KVQ_BEAM) &&
           (p->search != KVQ_BEAM || (p->beam_width >= 1 && p->beam_width <= KVQ_MAX_BEAM)) &&
           p->n_tensors >= 1 && p->n_tensors <= KVQ_MAX_TENSORS;
}

// Validate tensors against the plan and build the kernels' geometry.
kvq_status make_geom(const kvq_plan* p, const kvq_tensor* t, int32_t nt, kvq::Geom& g) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (!t) return fail(KVQ_EINVAL, "null tensor array");
    if (nt != p->n_tensors) return fail(KVQ_EINVAL, "plan is for %d tensors, got %d", p->n_tensors, nt);
    memset(&g, 0, sizeof g);
    g.contig = 1;
    for (int i = 0; i < nt; ++i) {
        if (!t[i].data) return fail(KVQ_EINVAL, "tensor %d: null data", i);
        if (t[i].dtype != p->dtype) return fail(KVQ_EINVAL, "tensor %d: dtype differs from plan", i);
        for (int d = 0; d < 4; ++d) {
            if (t[i].shape[d] != p->shape[i][d])
                return fail(KVQ_EINVAL, "tensor %d: shape differs from plan", i);
            if (t[i].stride[d] <= 0) return fail(KVQ_EINVAL, "tensor %d: non-positive stride", i);
        }
        g.data[i] = t[i].data;
        for (int d = 0; d < 4; ++d) g.stride[i][d] = t[i].stride[d];
        if (!(t[i].stride[3] == 1 && t[i].stride[2] == p->dims_per_block)) g.contig = 0;
    }
    g.nb0 = p->tensor_blocks[0];
    g.heads = (int32_t)p->shape[0][1];
    g.chunks = (int32_t)(p->shape[0][2] / p->tokens_per_block);
    g.groups = (int32_t)(p->shape[0][3] / p->dims_per_block);
    g.Tb = p->tokens_per_block;
    g.Db = p->dims_per_block;
    g.n = p->d_block;
    g.dtype = p->dtype;
    return KVQ_OK;
}

// The sort-free fp16 kernel covers s = 16 blocks of 4096 contiguous entries
// (whole head_dim rows, fully contiguous tensors, 16-byte aligned).
bool fast_fp16_path(const kvq_plan* p, const kvq_tensor* t, int32_t nt) {
    if (getenv("KVQ_FORCE_GENERIC")) return false;
    if (p->dtype != KVQ_F16 || p->s != 16 || p->d_block != 4096 || p->search != KVQ_GRIDS) return false;
    for (int i = 0; i < nt; ++i) {
        const int64_t* sh = t[i].shape;
        const int64_t* st = t[i].stride;
        if (p->dims_per_block != sh[3]) return false;
        if (st[3] != 1 || st[2] != sh[3] || st[1] != sh[2] * sh[3] || st[0] != sh[1] * sh[2] * sh[3])
            return false;
        if (((uintptr_t)t[i].data) & 15u) return false;
    }
    return true;
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status st) {
    switch (st) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_EINVAL: return "KVQ_EINVAL: invalid argument";
    case KVQ_EINFEASIBLE: return "KVQ_EINFEASIBLE: budget below the least-entropy allocation";
    case KVQ_ENONFINITE: return "KVQ_ENONFINITE: NaN or Inf in the KV input";
    case KVQ_ENOSPC: return "KVQ_ENOSPC: output capacity too small";
    case KVQ_EHIP: return "KVQ_EHIP: HIP runtime error";
    default: return "unknown kvq status";
    }
}

const char* kvq_last_error(void) { return g_err.c_str(); }

kvq_status kvq_plan_blocks(const kvq_tensor* t, int32_t nt, const kvq_block_spec* spec, kvq_plan* out) {
    if (!t || !spec || !out) return fail(KVQ_EINVAL, "null argument");
    if (nt < 1 || nt > KVQ_MAX_TENSORS) return fail(KVQ_EINVAL, "n_tensors must be 1 or 2");
    const int Tb = spec->tokens_per_block, Db = spec->dims_per_block;
    if (Tb <= 0 || Db <= 0) return fail(KVQ_EINVAL, "block shape must be positive");
    const int64_t n = (int64_t)Tb * Db;
    if (n < 2 || n > KVQ_MAX_BLOCK) return fail(KVQ_EINVAL, "block of %lld entries (need 2..4096)", (long long)n);
    if (spec->s < 2 || spec->s > KVQ_MAX_S) return fail(KVQ_EINVAL, "s=%d outside 2..16", spec->s);
    if (spec->search != KVQ_GRIDS && spec->search != KVQ_EXACT_DP && spec->search != KVQ_BEAM)
        return fail(KVQ_EINVAL, "unknown search mode %d", spec->search);
    if (spec->search == KVQ_BEAM && (spec->beam_width < 1 || spec->beam_width > KVQ_MAX_BEAM))
        return fail(KVQ_EINVAL, "beam_width=%d outside 1..%d", spec->beam_width, KVQ_MAX_BEAM);
    if (spec->search != KVQ_GRIDS && (spec->alphabet_m < 2 || spec->alphabet_m > KVQ_MAX_ALPHABET))
        return fail(KVQ_EINVAL, "alphabet_m=%d outside 2..%d", spec->alphabet_m, KVQ_MAX_ALPHABET);
    kvq_plan p;
    memset(&p, 0, sizeof p);
    p.dtype = t[0].dtype;
    if (p.dtype != KVQ_F16 && p.dtype != KVQ_F32) return fail(KVQ_EINVAL, "dtype must be KVQ_F16 or KVQ_F32");
    int64_t R = 0;
    for (int i = 0; i < nt; ++i) {
        if (t[i].dtype != p.dtype) return fail(KVQ_EINVAL, "tensors must share a dtype");
        for (int d = 0; d < 4; ++d)
            if (t[i].shape[d] <= 0) return fail(KVQ_EINVAL, "tensor %d: empty or negative dimension", i);
        for (int d = 0; d < 4; ++d) {
            if (t[i].shape[d] != t[0].shape[d]) return fail(KVQ_EINVAL, "tensors must share a shape");
            if (t[i].stride[d] <= 0) return fail(KVQ_EINVAL, "tensor %d: non-positive stride", i);
            p.shape[i][d] = t[i].shape[d];
        }
        if (t[i].shape[2] % Tb) return fail(KVQ_EINVAL, "tokens %lld not a multiple of %d", (long long)t[i].shape[2], Tb);
        if (t[i].shape[3] % Db) return fail(KVQ_EINVAL, "dim %lld not a multiple of %d", (long long)t[i].shape[3], Db);
        const int64_t nb = t[i].shape[0] * t[i].shape[1] * (t[i].shape[2] / Tb) * (t[i].shape[3] / Db);
        p.tensor_blocks[i] = nb;
        R += nb;
    }
    if (R >= (int64_t)1 << 31) return fail(KVQ_EINVAL, "too many blocks (%lld)", (long long)R);
    if (t[0].shape[1] >= ((int64_t)1 << 31) || t[0].shape[2] / Tb >= ((int64_t)1 << 31))
        return fail(KVQ_EINVAL, "dimension too large");
    p.n_blocks = R;
    p.n_entries = R * n;
    p.d_block = (int32_t)n;
    p.s = spec->s;
    p.search = spec->search;
    p.alphabet_m = spec->search != KVQ_GRIDS ? spec->alphabet_m : 0;
    p.beam_width = spec->search == KVQ_BEAM ? spec->beam_width : 0;
    p.n_tensors = nt;
    p.tokens_per_block = Tb;
    p.dims_per_block = Db;
    int max_levels;
    if (p.search == KVQ_GRIDS) {
        p.n_cand = 1 + 2 * (p.s - 2);
        p.n_stats = distinct_quantile_ranks((int)n, p.s, nullptr);
        if (p.n_stats > kvq::kMaxStats) return fail(KVQ_EINVAL, "too many order statistics");
        p.D_bytes = (size_t)R * p.n_cand * sizeof(double);
        p.H_bytes = p.D_bytes;
        max_levels = p.s;
    } else {
        p.n_cand = kvq::n_pairs(p.alphabet_m);
        p.n_stats = p.alphabet_m;
        p.D_bytes = (size_t)R * p.n_cand * sizeof(double);
        p.H_bytes = 2 * p.D_bytes;
        max_levels = p.s < p.alphabet_m ? p.s : p.alphabet_m;
    }
    p.stats_bytes = (size_t)R * p.n_stats * sizeof(float);
    p.choice_bytes = (size_t)R * sizeof(int32_t);
    p.codebook_bytes = (size_t)R * p.s * sizeof(float);
    p.m_bytes = (size_t)R;
    p.offsets_bytes = (size_t)(R + 1) * sizeof(uint64_t);
    p.workspace_bytes = kvq::ws_pool_offset(R) + (size_t)kvq::kGreedyPool * 8;
    p.max_code_words = (uint64_t)R * (((uint64_t)n * kvq::code_width(max_levels) + 31) / 32);
    // fixed point for exact rate sums: total <= n_entries * log2(levels) bits
    const double max_rate = (double)p.n_entries * (double)kvq::code_width(max_levels) + 1.0;
    int shift = 62 - (int)ceil(log2(max_rate));
    p.rate_shift = shift > 40 ? 40 : (shift < 0 ? 0 : shift);
    *out = p;
    return ok();
}

namespace {

// ---- the steps of the three admission calls, shared by kvq_admit ----

kvq_status eval_enqueue(const kvq_plan* p, const kvq_tensor* t, int32_t nt, const kvq::Geom& g, double* D,
                        double* H, float* stats, void* workspace, hipStream_t s) {
    hipError_t e = kvq::launch_ws_reset(workspace, s);
    if (e != hipSuccess) return hip_fail(e, "ws_reset");
    if (p->search == KVQ_GRIDS) {
        kvq::RankTable rt;
        rank_table(*p, rt);
        if (fast_fp16_path(p, t, nt))
            e = kvq::launch_eval16(t[0].data, nt > 1 ? t[1].data : t[0].data, p->tensor_blocks[0],
                                   p->n_blocks, rt, D, H, stats, workspace, s);
        else
            e = kvq::launch_eval_grids(g, p->n_blocks, p->s, rt, D, H, stats, workspace, s);
    } else {
        e = kvq::launch_eval_alphabet(g, p->n_blocks, p->alphabet_m, D, H, stats, workspace, s);
    }
    if (e != hipSuccess) return hip_fail(e, "eval launch");
    return ok();
}

kvq_status solve_check(const kvq_plan* p, const double* D, const double* H, const double* weight,
                       const float* stats, double B, int32_t mode, int32_t iters, double eta,
                       const double* lambda_io, const double* rate_out, const int32_t* choice,
                       const float* codebook, const uint8_t* m, const uint64_t* word_off,
                       const void* workspace) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (weight && p->search != KVQ_GRIDS) return fail(KVQ_EINVAL, "distortion weights need KVQ_GRIDS");
    if (!D || !H || !stats || !choice || !codebook || !m || !word_off || !workspace)
        return fail(KVQ_EINVAL, "null device pointer");
    if (!lambda_io || !rate_out) return fail(KVQ_EINVAL, "null host pointer");
    if (mode != KVQ_BISECT && mode != KVQ_SUBGRAD && mode != KVQ_BISECT_GREEDY)
        return fail(KVQ_EINVAL, "unknown mode %d", mode);
    if (mode == KVQ_BISECT_GREEDY && p->search != KVQ_GRIDS)
        return fail(KVQ_EINVAL, "the greedy post-pass needs KVQ_GRIDS");
    if (!isfinite(B) || B < 0.0) return fail(KVQ_EINVAL, "budget must be finite and >= 0");
    if (mode != KVQ_SUBGRAD && (iters < 0 || iters > 63)) return fail(KVQ_EINVAL, "iters must be 0..63");
    const double lam_in = *lambda_io;
    if (mode == KVQ_SUBGRAD && (!isfinite(lam_in) || lam_in < 0.0 || !isfinite(eta)))
        return fail(KVQ_EINVAL, "subgradient needs finite lambda >= 0 and finite eta");
    return ok();
}

// Where the solve's result will be found once the stream has reached it.
struct SolveState {
    kvq::SolveOut* out;  // pinned host buffer written by the last kernel, if `direct`
    bool direct;
    bool staging;        // read-backs may use the pinned staging buffer
};

kvq_status solve_enqueue(const kvq_plan* p, const double* D, const double* H, const double* weight,
                         const float* stats, double B, int32_t mode, int32_t iters, double lam_in,
                         int32_t* choice, float* codebook, uint8_t* m, uint64_t* word_off, void* workspace,
                         hipStream_t s, SolveState& ss, bool staging = true) {
    kvq::RankTable rt;
    rank_table(*p, rt);
    void* dev_out = nullptr;
    ss.out = staging ? static_cast<kvq::SolveOut*>(kvq::staging_buffer(&dev_out)) : nullptr;
    ss.direct = false;
    ss.staging = staging;
    const hipError_t e = kvq::launch_solve(*p, rt, D, H, weight, stats, B, mode, iters, lam_in, choice,
                                           codebook, m, word_off, workspace,
                                           ss.out ? static_cast<kvq::SolveOut*>(dev_out) : nullptr,
                                           &ss.direct, s, staging);
    if (e != hipSuccess) return hip_fail(e, "solve launch");
    return ok();
}

// Wait for the stream, read the solve's result and turn it into lambda,
// the modelled rate and a status.
kvq_status solve_result(const kvq_plan* p, double B, int32_t mode, double eta, double lam_in,
                        void* workspace, hipStream_t s, const SolveState& ss, double* lambda_io,
                        double* rate_out) {
    kvq::SolveOut hdr;
    hipError_t e;
    if (ss.direct) {
        // the last kernel wrote the result into the pinned buffer
        e = hipStreamSynchronize(s);
        if (e == hipSuccess) memcpy(&hdr, ss.out, sizeof hdr);
    } else {
        kvq::WsHeader full;
        e = kvq::read_back(&full, workspace, kvq::kWsHeaderReadBytes, s, ss.staging);
        hdr.status = full.status;
        hdr.err = full.err;
        hdr.pool_overflow = full.pool_overflow;
        hdr.lam_final = full.lam_final;
        hdr.rate_final = full.rate_final;
    }
    if (e != hipSuccess) return hip_fail(e, "status read-back");
    if (hdr.status & kvq::kStatusNonFinite) return fail(KVQ_ENONFINITE, "NaN or Inf among the KV entries");
    if (hdr.status & kvq::kStatusFusedStall)
        return fail(KVQ_EHIP, "one-launch admission: a block's offset look-back did not complete");
    if (hdr.err == KVQ_EINFEASIBLE)
        return fail(KVQ_EINFEASIBLE, "no lambda <= 2^64 brings the rate under %g bits/entry", B);
    if (hdr.err) return fail(KVQ_EINVAL, "solver state error %d", hdr.err);
    if (hdr.pool_overflow)
        return fail(KVQ_ENOSPC, "greedy post-pass: more than %u upgrades fit the slack", kvq::kGreedyPool);
    const double rbar = ldexp((double)hdr.rate_final, -p->rate_shift) / (double)p->n_entries;
    *rate_out = rbar;
    if (mode == KVQ_SUBGRAD) {
        const double nxt = lam_in + eta * (rbar - B);
        *lambda_io = nxt > 0.0 ? nxt : 0.0;
    } else {
        *lambda_io = hdr.lam_final;
    }
    return ok();
}

// Device address of `scratch` on the current device, looked up once per
// device (each device has its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

kvq_status noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EINVAL, "device %d outside 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(KVQ_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

// A one-launch admission's words buffer and the epoch of its last launch.
// Every launch on a buffer takes the next epoch; the buffer is cleared on
// the stream before its first launch and whenever the epochs start over, so
// no word of an earlier launch ever carries the current epoch.
struct FusedWords {
    uint64_t* words = nullptr;
    uint32_t epoch = 0;
};

kvq_status next_fused_epoch(FusedWords& fw, hipStream_t s, uint32_t* epoch) {
    if (fw.epoch == 0u || fw.epoch >= kvq::kFusedEpochMax) {
        const hipError_t e = kvq::launch_fused_words_clear(fw.words, s);
        if (e != hipSuccess) return hip_fail(e, "clearing the admission's published words");
        fw.epoch = 0u;
    }
    *epoch = ++fw.epoch;
    return KVQ_OK;
}

// kvq_admit: one words buffer per host thread and device, allocated on first
// use and kept until the process ends (a thread's calls wait for their
// result, so its launches never overlap).
kvq_status thread_fused_words(hipStream_t s, uint64_t** words, uint32_t* epoch) {
    thread_local FusedWords tl[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EINVAL, "device %d outside 0..%d", dev, kMaxDevices - 1);
    FusedWords& fw = tl[dev];
    if (!fw.words) {
        e = hipMalloc((void**)&fw.words, kvq::kFusedWordsBytes);
        if (e != hipSuccess) {
            fw.words = nullptr;
            return hip_fail(e, "hipMalloc (admission words)");
        }
        fw.epoch = 0u;
    }
    *words = fw.words;
    return next_fused_epoch(fw, s, epoch);
}

// kvq_admit_noalloc: the words at the end of the device's static scratch
// (calls that overlap on one device race, as for the rest of the scratch).
FusedWords g_scratch_words[kMaxDevices];

kvq_status scratch_fused_words(void* scratch_ptr, hipStream_t s, uint64_t** words, uint32_t* epoch) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EINVAL, "device %d outside 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    FusedWords& fw = g_scratch_words[dev];
    fw.words = reinterpret_cast<uint64_t*>(static_cast<char*>(scratch_ptr) + kvq::kNoAllocSolveBytes);
    *words = fw.words;
    return next_fused_epoch(fw, s, epoch);
}

// The admission step at a known multiplier (subgradient mode) on up to
// kFusedMaxBlocks fp16 blocks of 4096 contiguous entries with s = 16: one
// kernel scores, chooses, quantizes and packs, and the call waits once for
// its result.  Outputs are those of the three
// calls.
bool fused_admission(const kvq_plan* p, const kvq_tensor* t, int32_t nt, int32_t mode) {
    return mode == KVQ_SUBGRAD && p->n_blocks >= 1 && p->n_blocks <= kvq::kFusedMaxBlocks &&
           fast_fp16_path(p, t, nt);
}

kvq_status admit_fused(const kvq_plan* p, const kvq_tensor* t, int32_t nt, double* D, double* H, float* stats,
                       double B, double eta, double* lambda_io, double* rate_out, int32_t* choice,
                       float* codebook, uint8_t* m, uint64_t* word_off, uint64_t seed, uint32_t* codes,
                       void* ws, hipStream_t s, bool staging) {
    uint64_t* words = nullptr;
    uint32_t epoch = 0;
    kvq_status st = staging ? thread_fused_words(s, &words, &epoch) : scratch_fused_words(ws, s, &words, &epoch);
    if (st) return st;
    kvq::RankTable rt;
    rank_table(*p, rt);
    const double lam_in = *lambda_io;
    void* dev_out = nullptr;
    SolveState ss;
    ss.out = staging ? static_cast<kvq::SolveOut*>(kvq::staging_buffer(&dev_out)) : nullptr;
    ss.direct = ss.out != nullptr && dev_out != nullptr;
    ss.staging = staging;
    const hipError_t e = kvq::launch_admit_fused(t[0].data, nt > 1 ? t[1].data : t[0].data, p->tensor_blocks[0],
                                                 p->n_blocks, rt, lam_in, p->rate_shift, seed, D, H, stats,
                                                 choice, codebook, m, word_off, codes, ws, words, epoch,
                                                 ss.direct ? static_cast<kvq::SolveOut*>(dev_out) : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "one-launch admission");
    return solve_result(p, B, KVQ_SUBGRAD, eta, lam_in, ws, s, ss, lambda_io, rate_out);
}

kvq_status quantize_check(const kvq_plan* p, const float* codebook, const uint8_t* m, const uint64_t* word_off,
                          const uint32_t* codes, uint64_t cap) {
    if (!codebook || !m || !word_off || (!codes && p->max_code_words))
        return fail(KVQ_EINVAL, "null device pointer");
    if (cap < p->max_code_words)
        return fail(KVQ_ENOSPC, "codes capacity %llu words < plan.max_code_words %llu",
                    (unsigned long long)cap, (unsigned long long)p->max_code_words);
    return ok();
}

}  // namespace

kvq_status kvq_eval_candidates(const kvq_plan* p, const kvq_tensor* t, int32_t nt, double* D, double* H,
                               float* stats, void* workspace, hipStream_t s) {
    kvq::Geom g;
    kvq_status st = make_geom(p, t, nt, g);
    if (st) return st;
    if (!D || !H || !stats || !workspace) return fail(KVQ_EINVAL, "null output or workspace");
    return eval_enqueue(p, t, nt, g, D, H, stats, workspace, s);
}

kvq_status kvq_solve_lambda(const kvq_plan* p, const double* D, const double* H, const float* stats,
                            double B, int32_t mode, int32_t iters, double eta, double* lambda_io,
                            double* rate_out, int32_t* choice, float* codebook, uint8_t* m,
                            uint64_t* word_off, void* workspace, hipStream_t s) {
    return kvq_solve_lambda_weighted(p, D, H, nullptr, stats, B, mode, iters, eta, lambda_io, rate_out,
                                     choice, codebook, m, word_off, workspace, s);
}

kvq_status kvq_solve_lambda_weighted(const kvq_plan* p, const double* D, const double* H,
                                     const double* weight, const float* stats, double B, int32_t mode,
                                     int32_t iters, double eta, double* lambda_io, double* rate_out,
                                     int32_t* choice, float* codebook, uint8_t* m, uint64_t* word_off,
                                     void* workspace, hipStream_t s) {
    kvq_status st = solve_check(p, D, H, weight, stats, B, mode, iters, eta, lambda_io, rate_out, choice,
                                codebook, m, word_off, workspace);
    if (st) return st;
    const double lam_in = *lambda_io;
    SolveState ss;
    st = solve_enqueue(p, D, H, weight, stats, B, mode, iters, lam_in, choice, codebook, m, word_off,
                       workspace, s, ss);
    if (st) return st;
    return solve_result(p, B, mode, eta, lam_in, workspace, s, ss, lambda_io, rate_out);
}

kvq_status kvq_quantize_pack(const kvq_plan* p, const kvq_tensor* t, int32_t nt, const float* codebook,
                             const uint8_t* m, const uint64_t* word_off, uint64_t seed, uint32_t* codes,
                             uint64_t cap, hipStream_t s) {
    kvq::Geom g;
    kvq_status st = make_geom(p, t, nt, g);
    if (st) return st;
    st = quantize_check(p, codebook, m, word_off, codes, cap);
    if (st) return st;
    hipError_t e = kvq::launch_quantize(g, p->n_blocks, p->s, codebook, m, word_off, seed, codes, s);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return ok();
}

kvq_status kvq_admit(const kvq_plan* p, const kvq_tensor* t, int32_t nt, double* D, double* H, float* stats,
                     double B, int32_t mode, int32_t iters, double eta, double* lambda_io, double* rate_out,
                     int32_t* choice, float* codebook, uint8_t* m, uint64_t* word_off, uint64_t seed,
                     uint32_t* codes, uint64_t cap, void* workspace, hipStream_t s) {
    kvq::Geom g;
    kvq_status st = make_geom(p, t, nt, g);
    if (st) return st;
    if (!D || !H || !stats || !workspace) return fail(KVQ_EINVAL, "null output or workspace");
    if (mode == KVQ_BISECT_GREEDY) return fail(KVQ_EINVAL, "kvq_admit takes KVQ_BISECT or KVQ_SUBGRAD");
    st = solve_check(p, D, H, nullptr, stats, B, mode, iters, eta, lambda_io, rate_out, choice, codebook, m,
                     word_off, workspace);
    if (st) return st;
    st = quantize_check(p, codebook, m, word_off, codes, cap);
    if (st) return st;
    if (fused_admission(p, t, nt, mode))
        return admit_fused(p, t, nt, D, H, stats, B, eta, lambda_io, rate_out, choice, codebook, m, word_off, seed,
                           codes, workspace, s, /*staging=*/true);
    const double lam_in = *lambda_io;
    st = eval_enqueue(p, t, nt, g, D, H, stats, workspace, s);
    if (st) return st;
    SolveState ss;
    st = solve_enqueue(p, D, H, nullptr, stats, B, mode, iters, lam_in, choice, codebook, m, word_off,
                       workspace, s, ss);
    if (st) return st;
    // the codebooks and offsets stay on the device, so quantize_pack needs no
    // host round trip after the solve; one wait at the end returns lambda
    const hipError_t e = kvq::launch_quantize(g, p->n_blocks, p->s, codebook, m, word_off, seed, codes, s);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return solve_result(p, B, mode, eta, lam_in, workspace, s, ss, lambda_io, rate_out);
}

kvq_status kvq_admit_noalloc(const kvq_plan* p, const kvq_tensor* t, int32_t nt, double* D, double* H,
                             float* stats, double B, int32_t mode, int32_t iters, double eta, double* lambda_io,
                             double* rate_out, int32_t* choice, float* codebook, uint8_t* m, uint64_t* word_off,
                             uint64_t seed, uint32_t* codes, uint64_t cap, hipStream_t s) {
    kvq::Geom g;
    kvq_status st = make_geom(p, t, nt, g);
    if (st) return st;
    if (!D || !H || !stats) return fail(KVQ_EINVAL, "null output");
    if (mode != KVQ_BISECT && mode != KVQ_SUBGRAD)
        return fail(KVQ_EINVAL, "kvq_admit_noalloc takes KVQ_BISECT or KVQ_SUBGRAD");
    const size_t need = kvq::ws_pool_offset(p->n_blocks);
    if (need > kvq::kNoAllocSolveBytes)
        return fail(KVQ_ENOSPC, "%lld blocks need %zu bytes of solve scratch; the static scratch holds %zu "
                    "(at most 3668992 blocks)", (long long)p->n_blocks, need, kvq::kNoAllocSolveBytes);
    // every argument is checked before the scratch is touched
    int dummy = 0;
    st = solve_check(p, D, H, nullptr, stats, B, mode, iters, eta, lambda_io, rate_out, choice, codebook, m,
                     word_off, &dummy);
    if (st) return st;
    st = quantize_check(p, codebook, m, word_off, codes, cap);
    if (st) return st;
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st) return st;
    if (fused_admission(p, t, nt, mode))
        return admit_fused(p, t, nt, D, H, stats, B, eta, lambda_io, rate_out, choice, codebook, m, word_off, seed,
                           codes, ws, s, /*staging=*/false);
    const double lam_in = *lambda_io;
    // the scratch keeps the previous call's contents: eval's reset kernel
    // clears the status word and the solve's first kernel sets up the
    // header; the scan tile sums are written before they are read
    st = eval_enqueue(p, t, nt, g, D, H, stats, ws, s);
    if (st) return st;
    SolveState ss;
    st = solve_enqueue(p, D, H, nullptr, stats, B, mode, iters, lam_in, choice, codebook, m, word_off, ws, s, ss,
                       /*staging=*/false);
    if (st) return st;
    const hipError_t e = kvq::launch_quantize(g, p->n_blocks, p->s, codebook, m, word_off, seed, codes, s);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return solve_result(p, B, mode, eta, lam_in, ws, s, ss, lambda_io, rate_out);
}

kvq_status kvq_dequantize(const kvq_plan* p, const uint32_t* codes, const float* codebook, const uint8_t* m,
                          const uint64_t* word_off, float* xhat, hipStream_t s) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (!codebook || !m || !word_off || !xhat || (!codes && p->max_code_words))
        return fail(KVQ_EINVAL, "null device pointer");
    hipError_t e = kvq::launch_dequantize(p->n_blocks, p->d_block, p->s, codes, codebook, m, word_off, xhat, s);
    if (e != hipSuccess) return hip_fail(e, "dequantize launch");
    return ok();
}

kvq_status kvq_ans_sizes(const kvq_plan* p, uint64_t* scratch_bytes, uint64_t* stream_bytes) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (!scratch_bytes || !stream_bytes) return fail(KVQ_EINVAL, "null host pointer");
    const uint64_t b = 4u * p->max_code_words + (uint64_t)p->n_blocks * kvq::ans_margin_bytes(p->d_block);
    *scratch_bytes = b;
    *stream_bytes = b;
    return ok();
}

kvq_status kvq_ans_encode(const kvq_plan* p, const uint32_t* codes, const uint8_t* m,
                          const uint64_t* word_off, void* scratch, uint64_t scratch_bytes, void* stream,
                          uint64_t stream_bytes, uint64_t* block_off, void* workspace,
                          uint64_t* total_bytes_out, hipStream_t s) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (!m || !word_off || !scratch || !stream || !block_off || !workspace || (!codes && p->max_code_words))
        return fail(KVQ_EINVAL, "null device pointer");
    if (!total_bytes_out) return fail(KVQ_EINVAL, "null host pointer");
    uint64_t need = 0, need2 = 0;
    kvq_ans_sizes(p, &need, &need2);
    if (scratch_bytes < need || stream_bytes < need2)
        return fail(KVQ_ENOSPC, "entropy-coding buffers need %llu bytes each (kvq_ans_sizes)",
                    (unsigned long long)need);
    if ((((uintptr_t)scratch) | ((uintptr_t)stream)) & 3u) return fail(KVQ_EINVAL, "buffers must be 4-byte aligned");
    hipError_t e = kvq::launch_ws_reset(workspace, s);
    if (e != hipSuccess) return hip_fail(e, "ws_reset");
    e = kvq::launch_ans_encode(codes, m, word_off, p->n_blocks, p->d_block, p->s, (uint16_t*)scratch,
                               (uint8_t*)stream, block_off, workspace, s);
    if (e != hipSuccess) return hip_fail(e, "entropy-coding launch");
    kvq::WsHeader hdr;
    uint64_t total = 0;
    e = kvq::read_back(&hdr, workspace, kvq::kWsHeaderReadBytes, s);
    if (e == hipSuccess) e = kvq::read_back(&total, block_off + p->n_blocks, sizeof total, s);
    if (e != hipSuccess) return hip_fail(e, "entropy-coding read-back");
    if (hdr.status & kvq::kStatusAnsOverflow) return fail(KVQ_ENOSPC, "a coded block outgrew its scratch region");
    *total_bytes_out = total;
    return ok();
}

kvq_status kvq_ans_decode(const kvq_plan* p, const void* stream, const uint64_t* block_off,
                          const float* codebook, const uint8_t* m, float* xhat, void* workspace,
                          hipStream_t s) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (!stream || !block_off || !codebook || !m || !xhat || !workspace)
        return fail(KVQ_EINVAL, "null device pointer");
    if (((uintptr_t)stream) & 3u) return fail(KVQ_EINVAL, "stream must be 4-byte aligned");
    hipError_t e = kvq::launch_ans_decode((const uint8_t*)stream, block_off, codebook, m, p->n_blocks,
                                          p->d_block, p->s, xhat, workspace, s);
    if (e != hipSuccess) return hip_fail(e, "entropy-decoding launch");
    return ok();
}

static kvq_status attention_shape(const kvq_plan* p, int32_t q_heads, int& group) {
    if (!valid_plan(p)) return fail(KVQ_EINVAL, "invalid plan");
    if (p->n_tensors != 2) return fail(KVQ_EINVAL, "decode attention needs the K and V tensors");
    if (p->tokens_per_block != 32 || p->dims_per_block != 128 || p->shape[0][3] != 128)
        return fail(KVQ_EINVAL, "decode attention supports head x 32-token blocks of head_dim 128");
    for (int d = 0; d < 4; ++d)
        if (p->shape[1][d] != p->shape[0][d]) return fail(KVQ_EINVAL, "K and V must have the same shape");
    const int64_t heads = p->shape[0][1];
    if (p->shape[0][0] > 65535 || heads > 65535)
        return fail(KVQ_EINVAL, "decode attention takes at most 65535 outer slices and KV heads");
    if (q_heads <= 0 || q_heads % heads) return fail(KVQ_EINVAL, "query heads must be a multiple of KV heads");
    group = (int)(q_heads / heads);
    return ok();
}

kvq_status kvq_decode_attention_workspace(const kvq_plan* p, int32_t q_heads, uint64_t* bytes) {
    int group = 0;
    kvq_status st = attention_shape(p, q_heads, group);
    if (st) return st;
    if (!bytes) return fail(KVQ_EINVAL, "null host pointer");
    *bytes = kvq::attn_workspace_bytes(p->shape[0][0], (int)p->shape[0][1], (int)(p->shape[0][2] / 32), group);
    return ok();
}

kvq_status kvq_decode_attention(const kvq_plan* p, const uint32_t* codes, const float* codebook,
                                const uint8_t* m, const uint64_t* word_off, const float* q,
                                int32_t q_heads, float scale, float* out, void* work,
                                uint64_t work_bytes, hipStream_t s) {
    int group = 0;
    kvq_status st = attention_shape(p, q_heads, group);
    if (st) return st;
    if (!codebook || !m || !word_off || !q || !out || !work || (!codes && p->max_code_words))
        return fail(KVQ_EINVAL, "null device pointer");
    if (!isfinite(scale)) return fail(KVQ_EINVAL, "scale must be finite");
    uint64_t need = 0;
    kvq_decode_attention_workspace(p, q_heads, &need);
    if (work_bytes < need) return fail(KVQ_ENOSPC, "attention workspace needs %llu bytes", (unsigned long long)need);
    hipError_t e = kvq::launch_decode_attention(codes, codebook, m, word_off, p->tensor_blocks[0], p->shape[0][0],
                                                (int)p->shape[0][1], (int)(p->shape[0][2] / 32), p->s, group, q,
                                                scale, out, work, s);
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
    return ok();
}

}  // extern "C"
