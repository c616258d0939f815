// Host side of the C ABI declared in include/gdr.h: argument validation,
// workspace plan, and the stage sequence on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "gdr.h"
#include "gdr_fp16.hpp"
#include "gdr_launch.hpp"

namespace {

thread_local char g_err[512] = "";

gdr_status_t fail(gdr_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gdr_status_t fail(gdr_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    int64_t Ttot;
    int32_t nt_cap;
    size_t off_seq, off_start, off_len, off_first, off_R16, off_T16, off_P16, off_K16, off_Q16, off_G, off_A, off_W,
        off_U, off_KT, off_H, off_VN;
    size_t sz_T16, sz_R16, sz_K16, sz_A, sz_W, sz_U, sz_KT, sz_H, sz_VN;   // per chunk except A (whole)
    size_t production;         // bytes gdr_chunk_fwd needs
    size_t reference;          // bytes gdr_chunk_fwd_debug needs (five separate kernels)
};

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

gdr_status_t check_problem(const gdr_problem_t* p) {
    if (!p) return fail(GDR_ERR_NULL, "problem is NULL");
    if (p->batch < 1 || p->seq_len < 0)
        return fail(GDR_ERR_SHAPE, "batch must be >= 1 and seq_len >= 0 (got %lld, %lld)",
                    (long long)p->batch, (long long)p->seq_len);
    if (p->num_qk_heads < 1 || p->num_v_heads < 1 || p->num_v_heads % p->num_qk_heads != 0)
        return fail(GDR_ERR_SHAPE, "num_v_heads (%d) must be a positive multiple of num_qk_heads (%d)",
                    p->num_v_heads, p->num_qk_heads);
    if (p->num_v_heads > 65535 || p->num_qk_heads > 65535)
        return fail(GDR_ERR_SHAPE, "more than 65535 heads");
    if (p->head_dim_qk < 1 || p->head_dim_v < 1)
        return fail(GDR_ERR_SHAPE, "head dims must be positive");
    if (p->io_dtype != GDR_F32 && p->io_dtype != GDR_BF16)
        return fail(GDR_ERR_DTYPE, "unknown io_dtype %d", p->io_dtype);
    if (p->beta_dtype != p->io_dtype && p->beta_dtype != GDR_F32)
        return fail(GDR_ERR_DTYPE, "beta_dtype must equal io_dtype or be GDR_F32");
    if (p->out_dtype != p->io_dtype && p->out_dtype != GDR_F32)
        return fail(GDR_ERR_DTYPE, "out_dtype must equal io_dtype or be GDR_F32");
    if (!supported_dim(p->head_dim_qk) || !supported_dim(p->head_dim_v))
        return fail(GDR_ERR_UNSUPPORTED, "head dims (%d, %d) not in {32, 64, 128}", p->head_dim_qk, p->head_dim_v);
    if (p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64)
        return fail(GDR_ERR_UNSUPPORTED, "chunk_size %d not supported (16, 32 or 64)", p->chunk_size);
    if (p->num_seqs < 0) return fail(GDR_ERR_SHAPE, "num_seqs must be >= 0");
    const int64_t Ttot = p->batch * p->seq_len;
    if (p->seq_len > ((int64_t)1 << 31) - 1 || Ttot > ((int64_t)1 << 31) - 1 - 64)
        return fail(GDR_ERR_SHAPE, "total tokens %lld exceed the int32 token index", (long long)Ttot);
    return GDR_OK;
}

gdr_status_t check_seqlens(const gdr_problem_t* p, const int32_t* cu, bool varlen) {
    if (!varlen) {
        if (p->num_seqs != p->batch)
            return fail(GDR_ERR_SHAPE, "num_seqs (%d) must equal batch (%lld) without cu_seqlens", p->num_seqs,
                        (long long)p->batch);
        return GDR_OK;
    }
    if (p->batch != 1) return fail(GDR_ERR_SEQLENS, "cu_seqlens requires batch == 1");
    if (p->num_seqs < 1) return fail(GDR_ERR_SEQLENS, "cu_seqlens needs num_seqs >= 1");
    if (!cu) return GDR_OK;   // device-only copy cannot be checked on the host
    if (cu[0] != 0) return fail(GDR_ERR_SEQLENS, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int32_t n = 0; n < p->num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return fail(GDR_ERR_SEQLENS, "cu_seqlens decreases at %d", n);
    if ((int64_t)cu[p->num_seqs] != p->seq_len)
        return fail(GDR_ERR_SEQLENS, "cu_seqlens[N] = %d but seq_len = %lld", cu[p->num_seqs], (long long)p->seq_len);
    return GDR_OK;
}

// The fp16 path runs for bf16 inputs with C = 64; everything else runs the
// five kernels, whose production workspace holds their intermediates too.
bool fused_path(const gdr_problem_t* p) { return p->io_dtype == GDR_BF16 && p->chunk_size == 64; }

// Workspace regions, 256-byte aligned, in this order: the chunk table; on the
// fp16 path its decay rows, T and score fragments and the fp16 K and Q tiles
// (the production workspace ends there); then the five-kernel path's gate sums and intermediates (its
// production workspace, and the debug entry point's for every problem).
Plan make_plan(const gdr_problem_t* p) {
    Plan pl;
    pl.Ttot = p->batch * p->seq_len;
    const size_t C = (size_t)p->chunk_size;
    const size_t CP = C < 32 ? 32 : C;             // chunk positions padded to whole 32-position pairs
    int64_t cap = pl.Ttot / (int64_t)C + p->num_seqs;
    if (cap < 1) cap = 1;
    pl.nt_cap = (int32_t)cap;
    const size_t es = p->io_dtype == GDR_BF16 ? 2 : 4;
    const size_t Nv = p->num_v_heads, Nk = p->num_qk_heads, dk = p->head_dim_qk, dv = p->head_dim_v;
    const size_t T = (size_t)(pl.Ttot > 0 ? pl.Ttot : 1);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    pl.off_seq = take(cap * 4);
    pl.off_start = take(cap * 4);
    pl.off_len = take(cap * 4);
    pl.off_first = take(((size_t)p->num_seqs + 1) * 4);
    const bool fused = fused_path(p);
    pl.sz_R16 = fused ? Nv * 2 * 64 * 4 : 0;      // exp(G), exp(G_last - G) per position
    pl.sz_T16 = fused ? Nv * gdr::kPackedPairs * 2 : 0;   // six fp16 pair fragments, two of them halved
    pl.off_R16 = take(cap * pl.sz_R16);
    pl.off_T16 = take(cap * pl.sz_T16);
    pl.off_P16 = take(cap * pl.sz_T16);
    pl.sz_K16 = fused ? Nk * 64 * dk * 2 : 0;     // fp16 K (and Q) tiles
    pl.off_K16 = take(cap * pl.sz_K16);
    pl.off_Q16 = take(cap * pl.sz_K16);
    const size_t fused_end = off;
    pl.off_G = take(T * Nv * 4);
    pl.sz_A = T * Nv * C * 4;
    pl.off_A = take(pl.sz_A);
    pl.sz_W = Nv * C * dk * 4;             // per chunk
    pl.off_W = take(cap * pl.sz_W);
    pl.sz_U = Nv * C * dv * 4;
    pl.off_U = take(cap * pl.sz_U);
    pl.sz_KT = Nk * CP * dk * es;
    pl.off_KT = take(cap * pl.sz_KT);
    pl.sz_H = Nv * dk * dv * 4;
    pl.off_H = take(cap * pl.sz_H);
    pl.sz_VN = Nv * CP * dv * 4;
    pl.off_VN = take(cap * pl.sz_VN);
    pl.reference = off;
    pl.production = fused ? fused_end : off;
    return pl;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// Segment-parallel state passing. Automatic choice (segment_chunks == 0): when
// the serial state pass has fewer than 64 workgroups (sequences x value heads x
// 16-column dv tiles), each sequence is cut into up to 256 / that many
// segments, so that the segmented passes fill the 256 compute units once;
// otherwise the serial pass runs (fewer than four segments per sequence do not
// repay the two extra passes).
int32_t auto_segments_per_seq(const gdr_problem_t* p) {
    const int64_t w0 = (int64_t)p->num_seqs * p->num_v_heads * (p->head_dim_v / 16);
    if (w0 <= 0 || w0 >= 64) return 1;
    return (int32_t)(256 / w0);
}

// Upper bound on the segment count for any cu_seqlens with this problem's
// num_seqs and total length.
int64_t segment_bound(const gdr_problem_t* p, int32_t seg_chunks) {
    if (seg_chunks > 0) return make_plan(p).nt_cap / seg_chunks + p->num_seqs;
    const int32_t per_seq = auto_segments_per_seq(p);
    return per_seq > 1 ? (int64_t)p->num_seqs * per_seq : 0;   // 0: the serial pass runs
}

struct SegPlan {
    size_t off_first, off_seqseg, off_Sloc, off_M, off_Sstart, end;
};

// Segment region, laid out after `base` bytes for `nseg` segments.
SegPlan make_seg_plan(const gdr_problem_t* p, size_t base, int64_t nseg) {
    SegPlan sp;
    const size_t Nv = p->num_v_heads, dk = p->head_dim_qk, dv = p->head_dim_v;
    size_t off = align256(base);
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    sp.off_first = take(((size_t)nseg + 1) * 4);
    sp.off_seqseg = take(((size_t)p->num_seqs + 1) * 4);
    sp.off_Sloc = take((size_t)nseg * Nv * dk * dv * 4);
    sp.off_M = take((size_t)nseg * Nv * dk * dk * 4);
    sp.off_Sstart = take((size_t)nseg * Nv * dk * dv * 4);
    sp.end = off;
    return sp;
}

// Chunks of every sequence (and the longest sequence's count) for this chunk size.
void count_chunks(const gdr_problem_t* p, const int32_t* cu_host, int64_t* nt, int64_t* max_chunks) {
    const int64_t C = p->chunk_size;
    *nt = 0;
    *max_chunks = 0;
    for (int32_t n = 0; n < p->num_seqs; ++n) {
        const int64_t len = cu_host ? (int64_t)cu_host[n + 1] - cu_host[n] : p->seq_len;
        *nt += (len + C - 1) / C;
        *max_chunks = (len + C - 1) / C > *max_chunks ? (len + C - 1) / C : *max_chunks;
    }
}

// Launch arguments of the forward pipeline over the workspace regions of `pl`.
gdr::LaunchArgs fill_args(const gdr_problem_t* p, const Plan& pl, int64_t nt, const void* q, const void* k,
                          const void* v, const float* g, const void* beta, float scale, const float* S0,
                          const int32_t* cu_dev, void* o, float* ST, char* w, bool reference, void* stream) {
    gdr::LaunchArgs a;
    a.bf16 = p->io_dtype == GDR_BF16;
    a.dk = p->head_dim_qk;
    a.dv = p->head_dim_v;
    a.C = p->chunk_size;
    a.Nk = p->num_qk_heads;
    a.Nv = p->num_v_heads;
    a.N = p->num_seqs;
    a.T_row = p->seq_len;
    a.Ttot = p->batch * p->seq_len;
    a.nt = (int32_t)nt;
    a.nt_cap = pl.nt_cap;
    a.q = q; a.k = k; a.v = v; a.beta = beta;
    a.beta_f32 = p->beta_dtype == GDR_F32;
    a.out_f32 = p->out_dtype == GDR_F32;
    a.g = g; a.S0 = S0; a.scale = scale;
    a.cu_dev = cu_dev;
    a.o = o; a.ST = ST;
    a.chunk_seq = reinterpret_cast<int32_t*>(w + pl.off_seq);
    a.chunk_start = reinterpret_cast<int32_t*>(w + pl.off_start);
    a.chunk_len = reinterpret_cast<int32_t*>(w + pl.off_len);
    a.seq_first = reinterpret_cast<int32_t*>(w + pl.off_first);
    a.G = reinterpret_cast<float*>(w + pl.off_G);
    a.A = w + pl.off_A; a.W = w + pl.off_W; a.U = w + pl.off_U; a.KT = w + pl.off_KT;
    a.H = w + pl.off_H; a.VN = w + pl.off_VN;
    a.T16 = pl.sz_T16 ? w + pl.off_T16 : nullptr;
    a.P16 = pl.sz_T16 ? w + pl.off_P16 : nullptr;
    a.R16 = pl.sz_R16 ? reinterpret_cast<float*>(w + pl.off_R16) : nullptr;
    a.K16 = pl.sz_K16 ? w + pl.off_K16 : nullptr;
    a.Q16 = pl.sz_K16 ? w + pl.off_Q16 : nullptr;
    a.reference = reference;
    a.prep_only = false;
    a.states16 = false;
    a.nseg = 0;
    a.seg_chunks = 0;
    a.seg_first = a.seq_seg = nullptr;
    a.Sloc = a.Mseg = a.Sstart = nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    return a;
}

// Checks shared by the chunked entry points: problem, offsets, required inputs, alignment.
gdr_status_t check_inputs(const gdr_problem_t* p, const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* S0, const int32_t* cu_dev, const int32_t* cu_host,
                          void* ws) {
    gdr_status_t st = check_problem(p);
    if (st != GDR_OK) return st;
    if ((cu_dev == nullptr) != (cu_host == nullptr))
        return fail(GDR_ERR_NULL, "cu_seqlens_dev and cu_seqlens_host must both be given or both be NULL");
    st = check_seqlens(p, cu_host, cu_host != nullptr);
    if (st != GDR_OK) return st;
    const int64_t Ttot = p->batch * p->seq_len;
    if (Ttot > 0 && (!q || !k || !v || !beta))
        return fail(GDR_ERR_NULL, "q, k, v and beta are required");
    const void* ptrs[] = {q, k, v, beta, g, S0};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return fail(GDR_ERR_SHAPE, "tensor base address not 16-byte aligned");
    if (!ws) return fail(GDR_ERR_WORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws & 255) != 0) return fail(GDR_ERR_WORKSPACE, "workspace not 256-byte aligned");
    return GDR_OK;
}

// Segments of the backward's forward recompute: its state pass runs one
// wavefront per (sequence, value head, 16 dv columns); the sequences are cut
// into up to 2048 / (that many) segments (segment-parallel state passing), so
// that the recompute's serial pass has about 2048 wavefronts.
int32_t bwd_segments_per_seq(const gdr_problem_t* p) {
    const int64_t w0 = (int64_t)p->num_seqs * p->num_v_heads * (p->head_dim_v / 16);
    if (w0 <= 0 || w0 >= 1024) return 1;
    return (int32_t)(2048 / w0);
}

// Backward workspace: the five-kernel forward's regions, then the backward's
// own, then the recompute's segment region.
struct BwdPlan {
    size_t off_P, off_Hn, off_Vn, off_WT, off_dSout, off_dVn, off_dWs, off_dqv, off_dkv, end;
    SegPlan seg;
    int64_t seg_bound;
};

BwdPlan make_bwd_plan(const gdr_problem_t* p, const Plan& pl) {
    BwdPlan bp;
    const size_t C = p->chunk_size, cap = (size_t)pl.nt_cap;
    const size_t Nv = p->num_v_heads, dk = p->head_dim_qk, dv = p->head_dim_v;
    const size_t T = (size_t)(pl.Ttot > 0 ? pl.Ttot : 1);
    size_t off = align256(pl.reference);
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    bp.off_P = take(cap * Nv * C * C * 4);
    bp.off_Hn = take(cap * Nv * dk * dv * 4);
    bp.off_Vn = take(T * Nv * dv * 4);
    bp.off_WT = take(cap * Nv * dk * C * 4);
    bp.off_dSout = take(cap * Nv * dk * dv * 4);
    bp.off_dVn = take(T * Nv * dv * 4);
    bp.off_dWs = take(T * Nv * dk * 4);
    bp.off_dqv = take(T * Nv * dk * 4);
    bp.off_dkv = take(T * Nv * dk * 4);
    const int32_t per_seq = bwd_segments_per_seq(p);
    bp.seg_bound = per_seq > 1 ? (int64_t)p->num_seqs * per_seq : 0;
    bp.seg = make_seg_plan(p, off, bp.seg_bound);
    bp.end = bp.seg_bound > 0 ? bp.seg.end : off;
    return bp;
}

gdr_status_t run(const gdr_problem_t* p, const void* q, const void* k, const void* v, const float* g,
                 const void* beta, float scale, const float* S0, const int32_t* cu_dev, const int32_t* cu_host,
                 void* o, float* ST, void* ws, size_t ws_bytes, void* stream, hipEvent_t* events,
                 bool reference, Plan* plan_out, int32_t* nt_out, int32_t seg_req = -1) {
    if (p && p->batch * p->seq_len > 0 && !o) return fail(GDR_ERR_NULL, "o is required");
    if ((o && !aligned16(o)) || (ST && !aligned16(ST)))
        return fail(GDR_ERR_SHAPE, "tensor base address not 16-byte aligned");
    gdr_status_t st = check_inputs(p, q, k, v, g, beta, S0, cu_dev, cu_host, ws);
    if (st != GDR_OK) return st;
    Plan pl = make_plan(p);
    size_t need = reference ? pl.reference : pl.production;
    const int64_t C = p->chunk_size;
    int64_t nt = 0, max_chunks = 0;
    count_chunks(p, cu_host, &nt, &max_chunks);
    if (nt > pl.nt_cap) return fail(GDR_ERR_SEQLENS, "chunk count %lld exceeds capacity", (long long)nt);

    // segments: seg_req < 0 none, 0 automatic, > 0 chunks per segment; only a
    // split of some sequence into two or more segments takes the segmented passes
    int64_t seg_chunks = 0, nseg = 0;
    if (seg_req >= 0 && max_chunks > 1) {
        if (seg_req > 0) {
            seg_chunks = seg_req;
        } else {
            const int32_t per_seq = auto_segments_per_seq(p);
            if (per_seq > 1) seg_chunks = (max_chunks + per_seq - 1) / per_seq;
        }
        if (seg_chunks > 0 && seg_chunks < max_chunks) {
            for (int32_t n = 0; n < p->num_seqs; ++n) {
                const int64_t len = cu_host ? (int64_t)cu_host[n + 1] - cu_host[n] : p->seq_len;
                nseg += ((len + C - 1) / C + seg_chunks - 1) / seg_chunks;
            }
        } else {
            seg_chunks = 0;
        }
    }
    SegPlan sp{};
    if (nseg > 0) {
        sp = make_seg_plan(p, need, nseg);
        need = sp.end;
    }
    if (ws_bytes < need) return fail(GDR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);

    char* w = static_cast<char*>(ws);
    gdr::LaunchArgs a = fill_args(p, pl, nt, q, k, v, g, beta, scale, S0, cu_dev, o, ST, w, reference, stream);
    a.nseg = (int32_t)nseg;
    a.seg_chunks = (int32_t)seg_chunks;
    a.seg_first = nseg ? reinterpret_cast<int32_t*>(w + sp.off_first) : nullptr;
    a.seq_seg = nseg ? reinterpret_cast<int32_t*>(w + sp.off_seqseg) : nullptr;
    a.Sloc = nseg ? reinterpret_cast<float*>(w + sp.off_Sloc) : nullptr;
    a.Mseg = nseg ? reinterpret_cast<float*>(w + sp.off_M) : nullptr;
    a.Sstart = nseg ? reinterpret_cast<float*>(w + sp.off_Sstart) : nullptr;

    hipError_t e = gdr::launch_forward(a, events);
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    if (plan_out) *plan_out = pl;
    if (nt_out) *nt_out = (int32_t)nt;
    g_err[0] = '\0';
    return GDR_OK;
}

// ---------------------------------------------------------------- no-allocation scratch
// gdr_chunk_fwd_noalloc's workspace: a file-scope device array, one copy per GPU
// (the loader places it with the code object on every device the library runs
// on; it lives until the process ends). Host code never passes `scratch` itself
// to a kernel or a copy (on the host it is only a stand-in for the symbol): the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

gdr_status_t scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(GDR_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status_t gdr_validate(const gdr_problem_t* problem, const int32_t* cu_seqlens_host) {
    gdr_status_t st = check_problem(problem);
    if (st != GDR_OK) return st;
    st = check_seqlens(problem, cu_seqlens_host, cu_seqlens_host != nullptr);
    if (st == GDR_OK) g_err[0] = '\0';
    return st;
}

gdr_status_t gdr_chunk_fwd_workspace_size(const gdr_problem_t* problem, size_t* bytes) {
    if (!bytes) return fail(GDR_ERR_NULL, "bytes is NULL");
    gdr_status_t st = check_problem(problem);
    if (st != GDR_OK) return st;
    *bytes = make_plan(problem).production;
    return GDR_OK;
}

gdr_status_t gdr_chunk_fwd_debug_workspace_size(const gdr_problem_t* problem, size_t* bytes) {
    if (!bytes) return fail(GDR_ERR_NULL, "bytes is NULL");
    gdr_status_t st = check_problem(problem);
    if (st != GDR_OK) return st;
    *bytes = make_plan(problem).reference;
    return GDR_OK;
}

gdr_status_t gdr_chunk_fwd(const gdr_problem_t* p, const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, const float* initial_state, const int32_t* cu_dev,
                           const int32_t* cu_host, void* o, float* final_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return run(p, q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, o, final_state, workspace,
               workspace_bytes, stream, nullptr, false, nullptr, nullptr);
}

gdr_status_t gdr_chunk_fwd_noalloc(const gdr_problem_t* p, const void* q, const void* k, const void* v,
                                   const float* g, const void* beta, float scale, const float* initial_state,
                                   const int32_t* cu_dev, const int32_t* cu_host, void* o, float* final_state,
                                   void* stream) {
    gdr_status_t st = check_problem(p);
    if (st != GDR_OK) return st;
    const size_t need = make_plan(p).production;
    if (need > kNoAllocScratchBytes)
        return fail(GDR_ERR_WORKSPACE,
                    "problem needs %zu bytes of scratch; gdr_chunk_fwd_noalloc holds %zu per GPU "
                    "(use gdr_chunk_fwd with a caller workspace)", need, kNoAllocScratchBytes);
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != GDR_OK) return st;
    return run(p, q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, o, final_state, ws,
               kNoAllocScratchBytes, stream, nullptr, false, nullptr, nullptr);
}

size_t gdr_chunk_fwd_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

gdr_status_t gdr_chunk_fwd_debug(const gdr_problem_t* p, const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, float scale, const float* initial_state,
                                 const int32_t* cu_dev, const int32_t* cu_host, void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream, gdr_intermediates_t* dbg) {
    if (!dbg) return fail(GDR_ERR_NULL, "dbg is NULL");
    if (reinterpret_cast<uintptr_t>(dbg->T) % 16 || reinterpret_cast<uintptr_t>(dbg->P) % 16)
        return fail(GDR_ERR_SHAPE, "dbg->T and dbg->P must be 16-byte aligned");
    Plan pl;
    int32_t nt = 0;
    gdr_status_t st = run(p, q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, o, final_state, workspace,
                          workspace_bytes, stream, nullptr, true, &pl, &nt);
    if (st != GDR_OK) return st;
    dbg->num_chunks = nt;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* w = static_cast<const char*>(workspace);
    const size_t Ttot = (size_t)pl.Ttot;
    struct { void* dst; size_t off; size_t bytes; } copies[] = {
        {dbg->G, pl.off_G, Ttot * (size_t)p->num_v_heads * 4},
        {dbg->A, pl.off_A, Ttot > 0 ? pl.sz_A : 0},
        {dbg->W, pl.off_W, (size_t)nt * pl.sz_W},
        {dbg->U, pl.off_U, (size_t)nt * pl.sz_U},
        {dbg->KT, pl.off_KT, (size_t)nt * pl.sz_KT},
        {dbg->H, pl.off_H, (size_t)nt * pl.sz_H},
        {dbg->VN, pl.off_VN, (size_t)nt * pl.sz_VN},
        {dbg->R, pl.off_R16, (size_t)nt * pl.sz_R16},
    };
    for (auto& c : copies) {
        if (!c.dst || c.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(c.dst, w + c.off, c.bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return fail(GDR_ERR_HIP, "intermediate copy failed: %s", hipGetErrorString(e));
    }
    // T and P: the workspace holds the pair sets packed; the copies get all six fragments
    const struct { void* dst; size_t off; } pairs[] = {{dbg->T, pl.off_T16}, {dbg->P, pl.off_P16}};
    for (auto& c : pairs) {
        if (!c.dst || pl.sz_T16 == 0 || nt == 0) continue;
        hipError_t e = gdr::unpack_pairs16(w + c.off, c.dst, (int64_t)nt * p->num_v_heads, s);
        if (e != hipSuccess) return fail(GDR_ERR_HIP, "intermediate copy failed: %s", hipGetErrorString(e));
    }
    return GDR_OK;
}

gdr_status_t gdr_chunk_fwd_segmented_workspace_size(const gdr_problem_t* problem, int32_t segment_chunks,
                                                    size_t* bytes) {
    if (!bytes) return fail(GDR_ERR_NULL, "bytes is NULL");
    gdr_status_t st = check_problem(problem);
    if (st != GDR_OK) return st;
    if (segment_chunks < 0) return fail(GDR_ERR_SHAPE, "segment_chunks must be >= 0 (got %d)", segment_chunks);
    const size_t base = make_plan(problem).production;
    *bytes = make_seg_plan(problem, base, segment_bound(problem, segment_chunks)).end;
    return GDR_OK;
}

gdr_status_t gdr_chunk_fwd_segmented(const gdr_problem_t* p, const void* q, const void* k, const void* v,
                                     const float* g, const void* beta, float scale, const float* initial_state,
                                     const int32_t* cu_dev, const int32_t* cu_host, void* o, float* final_state,
                                     int32_t segment_chunks, void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* stage_events) {
    if (segment_chunks < 0) return fail(GDR_ERR_SHAPE, "segment_chunks must be >= 0 (got %d)", segment_chunks);
    hipEvent_t ev[GDR_NUM_STAGES + 1];
    if (stage_events)
        for (int i = 0; i <= GDR_NUM_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(stage_events[i]);
    return run(p, q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, o, final_state, workspace,
               workspace_bytes, stream, stage_events ? ev : nullptr, false, nullptr, nullptr, segment_chunks);
}

gdr_status_t gdr_chunk_bwd_workspace_size(const gdr_problem_t* problem, size_t* bytes) {
    if (!bytes) return fail(GDR_ERR_NULL, "bytes is NULL");
    gdr_status_t st = check_problem(problem);
    if (st != GDR_OK) return st;
    *bytes = make_bwd_plan(problem, make_plan(problem)).end;
    return GDR_OK;
}

gdr_status_t gdr_chunk_bwd(const gdr_problem_t* p, const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, const float* initial_state, const int32_t* cu_dev,
                           const int32_t* cu_host, const void* d_o, const float* d_final_state, float* dq,
                           float* dk, float* dv, float* dbeta, float* dg, float* d_initial_state, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* stage_events) {
    hipEvent_t ev[GDR_BWD_NUM_STAGES + 1];
    if (stage_events)
        for (int i = 0; i <= GDR_BWD_NUM_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(stage_events[i]);
    gdr_status_t st = check_inputs(p, q, k, v, g, beta, initial_state, cu_dev, cu_host, workspace);
    if (st != GDR_OK) return st;
    const int64_t Ttot = p->batch * p->seq_len;
    if (Ttot > 0 && (!d_o || !dq || !dk || !dv || !dbeta))
        return fail(GDR_ERR_NULL, "d_o, dq, dk, dv and dbeta are required");
    const void* ptrs[] = {d_o, d_final_state, dq, dk, dv, dbeta, dg, d_initial_state};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return fail(GDR_ERR_SHAPE, "tensor base address not 16-byte aligned");
    const Plan pl = make_plan(p);
    const BwdPlan bp = make_bwd_plan(p, pl);
    if (workspace_bytes < bp.end)
        return fail(GDR_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, bp.end);
    int64_t nt = 0, max_chunks = 0;
    count_chunks(p, cu_host, &nt, &max_chunks);
    if (nt > pl.nt_cap) return fail(GDR_ERR_SEQLENS, "chunk count %lld exceeds capacity", (long long)nt);

    char* w = static_cast<char*>(workspace);
    gdr::BackwardArgs b;
    // the recompute needs the chunk states and V_new, not o
    b.fwd = fill_args(p, pl, nt, q, k, v, g, beta, scale, initial_state, cu_dev, nullptr, nullptr, w, true,
                      stream);
    // bf16 with C = 64 and enough (sequence, head, column tile) units to fill
    // the GPU: the chunk states come from the fp16 chunk pass; otherwise from
    // the five-kernel state pass, segment-parallel when there are few units
    b.fwd.states16 = fused_path(p) && (int64_t)p->num_seqs * p->num_v_heads * (p->head_dim_v / 16) >= 128;
    const int32_t per_seq = b.fwd.states16 ? 1 : bwd_segments_per_seq(p);
    if (per_seq > 1 && max_chunks > 1) {
        const int64_t C = p->chunk_size;
        const int64_t seg_chunks = (max_chunks + per_seq - 1) / per_seq;
        int64_t nseg = 0;
        for (int32_t n = 0; n < p->num_seqs; ++n) {
            const int64_t len = cu_host ? (int64_t)cu_host[n + 1] - cu_host[n] : p->seq_len;
            nseg += ((len + C - 1) / C + seg_chunks - 1) / seg_chunks;
        }
        if (nseg > p->num_seqs && nseg <= bp.seg_bound) {
            const SegPlan sp = make_seg_plan(p, bp.seg.off_first, nseg);   // same start, nseg entries
            b.fwd.nseg = (int32_t)nseg;
            b.fwd.seg_chunks = (int32_t)seg_chunks;
            b.fwd.seg_first = reinterpret_cast<int32_t*>(w + sp.off_first);
            b.fwd.seq_seg = reinterpret_cast<int32_t*>(w + sp.off_seqseg);
            b.fwd.Sloc = reinterpret_cast<float*>(w + sp.off_Sloc);
            b.fwd.Mseg = reinterpret_cast<float*>(w + sp.off_M);
            b.fwd.Sstart = reinterpret_cast<float*>(w + sp.off_Sstart);
        }
    }
    b.d_o = d_o;
    b.do_f32 = p->out_dtype == GDR_F32;
    b.dST = d_final_state;
    b.dq = dq; b.dk = dk; b.dv = dv; b.dbeta = dbeta; b.dg = dg; b.dS0 = d_initial_state;
    auto f = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    b.P = f(bp.off_P); b.Hn = f(bp.off_Hn); b.Vn = f(bp.off_Vn); b.WT = f(bp.off_WT);
    b.dSout = f(bp.off_dSout); b.dVn = f(bp.off_dVn); b.dWs = f(bp.off_dWs);
    b.dqv = f(bp.off_dqv); b.dkv = f(bp.off_dkv);
    b.events = stage_events ? ev : nullptr;
    hipError_t e = gdr::launch_backward(b);
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return GDR_OK;
}

gdr_status_t gdr_chunk_fwd_timed(const gdr_problem_t* p, const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, float scale, const float* initial_state,
                                 const int32_t* cu_dev, const int32_t* cu_host, void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events) {
    if (!stage_events) return fail(GDR_ERR_NULL, "stage_events is NULL");
    hipEvent_t ev[GDR_NUM_STAGES + 1];
    for (int i = 0; i <= GDR_NUM_STAGES; ++i) ev[i] = static_cast<hipEvent_t>(stage_events[i]);
    return run(p, q, k, v, g, beta, scale, initial_state, cu_dev, cu_host, o, final_state, workspace,
               workspace_bytes, stream, ev, false, nullptr, nullptr);
}

const char* gdr_status_string(gdr_status_t s) {
    switch (s) {
        case GDR_OK: return "ok";
        case GDR_ERR_NULL: return "required pointer is NULL";
        case GDR_ERR_SHAPE: return "invalid shape or alignment";
        case GDR_ERR_DTYPE: return "invalid dtype";
        case GDR_ERR_UNSUPPORTED: return "unsupported by this build";
        case GDR_ERR_SEQLENS: return "invalid cu_seqlens";
        case GDR_ERR_WORKSPACE: return "workspace missing or too small";
        case GDR_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* gdr_last_error_message(void) { return g_err; }

gdr_status_t gdr_recurrent_fwd(const gdr_problem_t* p, const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float scale, const float* initial_state, const int32_t* cu_dev,
                               const int32_t* cu_host, int use_qk_l2norm, void* o, float* final_state,
                               void* stream) {
    if (!p) return fail(GDR_ERR_NULL, "problem is NULL");
    gdr_problem_t pc = *p;
    pc.chunk_size = 64;                        // not used by the token-by-token path
    gdr_status_t st = check_problem(&pc);
    if (st != GDR_OK) return st;
    if ((cu_dev == nullptr) != (cu_host == nullptr))
        return fail(GDR_ERR_NULL, "cu_seqlens_dev and cu_seqlens_host must both be given or both be NULL");
    st = check_seqlens(&pc, cu_host, cu_host != nullptr);
    if (st != GDR_OK) return st;
    const int64_t Ttot = pc.batch * pc.seq_len;
    if (Ttot > 0 && (!q || !k || !v || !beta || !o))
        return fail(GDR_ERR_NULL, "q, k, v, beta and o are required");
    const void* ptrs[] = {q, k, v, beta, g, initial_state, o, final_state};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return fail(GDR_ERR_SHAPE, "tensor base address not 16-byte aligned");
    gdr::RecurrentArgs a;
    a.bf16 = pc.io_dtype == GDR_BF16;
    a.dk = pc.head_dim_qk;
    a.dv = pc.head_dim_v;
    a.Nk = pc.num_qk_heads;
    a.Nv = pc.num_v_heads;
    a.N = pc.num_seqs;
    a.T_row = pc.seq_len;
    a.Ttot = Ttot;
    a.q = q; a.k = k; a.v = v; a.beta = beta;
    a.beta_f32 = pc.beta_dtype == GDR_F32;
    a.out_f32 = pc.out_dtype == GDR_F32;
    a.l2norm = use_qk_l2norm ? 1 : 0;
    a.g = g; a.S0 = initial_state; a.scale = scale;
    a.cu_dev = cu_dev;
    a.o = o; a.ST = final_state;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = gdr::launch_recurrent(a);
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return GDR_OK;
}

}  // extern "C"
