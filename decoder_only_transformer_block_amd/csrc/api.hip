// C ABI of libdtb: argument validation, buffer layouts and the launch
// sequences of block_forward / block_backward / attn_forward / attn_backward.
// Nothing here allocates device memory or synchronises the host (except the
// opt-in measurement helper dtb_timing_collect).
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "common.h"

namespace dtb {

// ---------------------------------------------------------------- errors ---
static thread_local char g_msg[256];

static thread_local hipError_t t_debug_err = hipSuccess;
static thread_local char t_debug_kernel[160];

int set_launch_error(hipError_t e, const char *what) {
    if (t_debug_kernel[0])
        snprintf(g_msg, sizeof g_msg, "kernel launch failed in %s (kernel %s): %s", what, t_debug_kernel,
                 hipGetErrorString(e));
    else
        snprintf(g_msg, sizeof g_msg, "kernel launch failed in %s: %s", what, hipGetErrorString(e));
    t_debug_kernel[0] = 0;
    return DTB_ELAUNCH;
}

// ---------------------------------------------------------------- debug ---
int g_debug_level = 0;

void debug_after_launch(hipStream_t s, const char *kernel) {
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        fprintf(stderr, "[dtb debug] %s failed: %s\n", kernel, hipGetErrorString(e));
        if (t_debug_err == hipSuccess) {
            t_debug_err = e;
            snprintf(t_debug_kernel, sizeof t_debug_kernel, "%s", kernel);
        }
    } else if (g_debug_level >= 2) {
        fprintf(stderr, "[dtb debug] %s ok\n", kernel);
    }
}

hipError_t last_error() {
    hipError_t e = hipGetLastError();
    if (t_debug_err != hipSuccess) {
        e = t_debug_err;
        t_debug_err = hipSuccess;
    }
    return e;
}

// ---------------------------------------------------------------- timing ---
bool g_timing_on = false;
static unsigned g_timing_mask = 0;  // bit c: class c is timed
struct TRec {
    hipEvent_t a, b;
    int cls;
    double flops, bytes;
};
static std::mutex g_tmu;
static std::vector<TRec> g_trec;
static std::vector<hipEvent_t> g_pool;
static std::vector<hipEvent_t> g_retired;  // stop events a later launch of their unit superseded
static bool g_unit_open = false;
static hipEvent_t g_unit_a = nullptr, g_unit_b = nullptr;
static dtb_timing g_tot[K_NCLASS];

static hipEvent_t ev_get() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// A timed unit is one or more launches on one stream (a GEMM and its split-K
// reduction, say).  Its start is the start of its first kernel and its end the
// end of its last, both taken from the kernels' own dispatch packets.
void timing_begin(hipStream_t, int cls) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_unit_open = ((g_timing_mask >> cls) & 1u) != 0;
    g_unit_a = g_unit_b = nullptr;
}

// While a class that block_backward launches is being timed, it runs on the
// caller's stream only, so the per-class times are not inflated by kernels of
// the side stream sharing the GPU.
static bool timing_serializes_backward() {
    const unsigned bwd = (1u << K_GEMM_DINP) | (1u << K_GEMM_DW) | (1u << K_ATTN_BWD) | (1u << K_ELEM);
    return g_timing_on && (g_timing_mask & bwd) != 0;
}

void timing_launch_events(hipEvent_t *start, hipEvent_t *stop) {
    std::lock_guard<std::mutex> lk(g_tmu);
    *start = *stop = nullptr;
    if (!g_unit_open) return;
    hipEvent_t b = ev_get();
    if (!b) return;
    if (!g_unit_a) {
        g_unit_a = ev_get();
        if (!g_unit_a) {
            g_pool.push_back(b);
            return;
        }
        *start = g_unit_a;
    }
    // an earlier stop event of this unit may still be pending on the device:
    // it is only reused after the next collection has waited for it
    if (g_unit_b) g_retired.push_back(g_unit_b);
    g_unit_b = b;
    *stop = b;
}

void timing_end(hipStream_t, int cls, double flops, double bytes) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_unit_open && g_unit_a && g_unit_b) {
        g_trec.push_back(TRec{g_unit_a, g_unit_b, cls, flops, bytes});
    } else {
        if (g_unit_a) g_retired.push_back(g_unit_a);
        if (g_unit_b) g_retired.push_back(g_unit_b);
    }
    g_unit_open = false;
    g_unit_a = g_unit_b = nullptr;
}

}  // namespace dtb

using namespace dtb;

extern "C" {

const char *dtb_version(void) { return "dtb 0.1 gfx950"; }

const char *dtb_strerror(int code) {
    switch (code) {
    case DTB_OK: return "ok";
    case DTB_EINVAL_SHAPE: return "invalid shape (C % NH, NH % NKV, unsupported head width, C or H not a multiple of 8, negative size or overflow)";
    case DTB_EINVAL_PTR: return "a required pointer is NULL or not 16-byte aligned";
    case DTB_EDTYPE: return "dtype must be DTB_F32 or DTB_BF16";
    case DTB_EINVAL_ENUM: return "unknown norm / mlp / rope selector";
    case DTB_ELAUNCH: return g_msg[0] ? g_msg : "kernel launch failed";
    default: return "unknown error code";
    }
}

int dtb_debug_enable(int level) {
    if (level < 0 || level > 2) return DTB_EINVAL_ENUM;
    g_debug_level = level;
    return DTB_OK;
}

int dtb_timing_enable(int class_mask) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing_mask = class_mask < 0 ? ~0u : (unsigned)class_mask;
    g_timing_on = g_timing_mask != 0;
    // events are created here, not on the launch path: creating them while
    // kernels are being enqueued made the host fall behind the GPU
    constexpr size_t kPool = 4096;
    while (g_timing_on && g_pool.size() + g_trec.size() * 2 + g_retired.size() < kPool) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) break;
        g_pool.push_back(e);
    }
    return DTB_OK;
}

int dtb_timing_collect(dtb_timing *out, int max_classes) {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &r : g_trec) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
            dtb_timing &t = g_tot[r.cls];
            t.ms += ms;
            t.flops += r.flops;
            t.bytes += r.bytes;
            t.launches += 1;
        }
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_trec.clear();
    for (hipEvent_t e : g_retired) {
        (void)hipEventSynchronize(e);
        g_pool.push_back(e);
    }
    g_retired.clear();
    int n = max_classes < K_NCLASS ? max_classes : K_NCLASS;
    for (int i = 0; i < n; i++) out[i] = g_tot[i];
    for (int i = 0; i < K_NCLASS; i++) g_tot[i] = dtb_timing{0, 0, 0, 0};
    return n;
}

}  // extern "C"

// ------------------------------------------------------------ validation ---
static bool hd_ok(int hd, int dtype) {
    if (dtype == DTB_BF16) return hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128;
    return hd == 4 || hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128;
}
static bool aligned(const void *p) { return ((uintptr_t)p & 15) == 0; }
static bool ptr_ok(const void *p) { return p && aligned(p); }

static int check_attn_shape(int B, int T, int C, int NH, int NKV, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (B < 0 || T < 0 || C <= 0 || NH <= 0 || NKV <= 0) return DTB_EINVAL_SHAPE;
    if (C % NH || NH % NKV) return DTB_EINVAL_SHAPE;
    if (!hd_ok(C / NH, dtype)) return DTB_EINVAL_SHAPE;
    long long QKV = (long long)C + 2LL * NKV * (C / NH);
    if ((long long)B * T * QKV >= (1LL << 40) || (long long)B * T >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    // the attention kernels address a sequence's rows by 32-bit byte offsets
    // from the sequence base (qkv rows of QKV elements, out / dout rows of C)
    const long long es = dtype == DTB_BF16 ? 2 : 4;
    if ((long long)T * QKV * es >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

struct Dims {
    long long BT;
    int hd, QKV, W, es;
};

static int check_cfg(const dtb_block_cfg *c, Dims *d) {
    if (!c) return DTB_EINVAL_PTR;
    int e = check_attn_shape(c->B, c->T, c->C, c->NH, c->NKV, c->dtype);
    if (e) return e;
    if (c->norm < 0 || c->norm > 2 || c->mlp < 0 || c->mlp > 2 || c->rope < 0 || c->rope > 1)
        return DTB_EINVAL_ENUM;
    if (c->H <= 0 || c->H % 8 || c->C % 8) return DTB_EINVAL_SHAPE;
    if (c->C > (c->dtype == DTB_BF16 ? 8192 : 4096)) return DTB_EINVAL_SHAPE;
    if (!(c->eps > 0.f)) return DTB_EINVAL_SHAPE;
    if (c->rope == DTB_ROPE_NEOX && !(c->rope_base > 0.f)) return DTB_EINVAL_SHAPE;
    d->BT = (long long)c->B * c->T;
    d->hd = c->C / c->NH;
    d->QKV = c->C + 2 * c->NKV * d->hd;
    d->W = c->mlp == DTB_MLP_SWIGLU ? 2 * c->H : c->H;
    d->es = c->dtype == DTB_BF16 ? 2 : 4;
    if (d->BT * (long long)(d->W > d->QKV ? d->W : d->QKV) >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

static size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

static void saved_layout(const dtb_block_cfg *c, const Dims &d, dtb_saved_layout *L) {
    size_t o = 0;
    auto take = [&](size_t bytes) {
        long long r = (long long)o;
        o += al(bytes);
        return r;
    };
    bool ln = c->norm == DTB_NORM_LAYER;
    L->n1 = take((size_t)d.BT * c->C * d.es);
    L->r1 = take((size_t)d.BT * 4);
    L->mu1 = ln ? take((size_t)d.BT * 4) : -1;
    L->qkv = take((size_t)d.BT * d.QKV * d.es);
    L->o = take((size_t)d.BT * c->C * d.es);
    L->lse = take((size_t)c->B * c->NH * c->T * 4);
    L->x2 = take((size_t)d.BT * c->C * d.es);
    L->n2 = take((size_t)d.BT * c->C * d.es);
    L->r2 = take((size_t)d.BT * 4);
    L->mu2 = ln ? take((size_t)d.BT * 4) : -1;
    L->up = take((size_t)d.BT * d.W * d.es);
    L->h = take((size_t)d.BT * c->H * d.es);
    L->total = (long long)o;
}

struct WsLayout {
    size_t cs, dh, dup, dn2, dx2, dO, dqkv, dn1, D, npart, bpart, gemm, total;
    int nparts, bparts;
    size_t gemm_bytes;
};

// The second stream of block_backward_overlap, owned by the caller (created
// and destroyed through dtb_overlap_create / dtb_overlap_destroy): the
// library itself keeps no stream or event between calls.
struct dtb_overlap_s {
    int device;
    hipStream_t s;
    hipEvent_t fork, join;
};

static void ws_layout(const dtb_block_cfg *c, const Dims &d, WsLayout *W) {
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t r = o;
        o += al(bytes);
        return r;
    };
    W->cs = take((size_t)c->T * (d.hd / 2) * 8);
    W->dh = take((size_t)d.BT * c->H * d.es);
    W->dup = take((size_t)d.BT * d.W * d.es);
    W->dn2 = take((size_t)d.BT * c->C * d.es);
    W->dx2 = take((size_t)d.BT * c->C * d.es);
    W->dO = take((size_t)d.BT * c->C * d.es);
    W->dqkv = take((size_t)d.BT * d.QKV * d.es);
    W->dn1 = take((size_t)d.BT * c->C * d.es);
    W->D = take((size_t)c->B * c->NH * c->T * 4 * 2);  // -D and -lse / scale
    W->nparts = norm_backward_parts(d.BT);
    W->npart = take(norm_backward_ws_bytes(d.BT, c->C));
    W->bparts = bias_grad_parts(d.BT);
    int maxn = d.QKV > d.W ? d.QKV : d.W;
    if (c->C > maxn) maxn = c->C;
    W->bpart = take((size_t)W->bparts * maxn * 4);
    int BT = (int)d.BT;
    size_t g = 0, t;
    t = gemm_ws_bytes(c->C, c->H, BT, c->dtype); if (t > g) g = t;
    t = gemm_ws_bytes(d.W, c->C, BT, c->dtype); if (t > g) g = t;
    t = gemm_ws_bytes(c->C, c->C, BT, c->dtype); if (t > g) g = t;
    t = gemm_ws_bytes(d.QKV, c->C, BT, c->dtype); if (t > g) g = t;
    W->gemm_bytes = g;
    W->gemm = take(g);
    W->total = o;
}

extern "C" {

size_t block_saved_bytes(const dtb_block_cfg *cfg) {
    Dims d;
    if (check_cfg(cfg, &d)) return 0;
    dtb_saved_layout L;
    saved_layout(cfg, d, &L);
    return (size_t)L.total;
}

int rope_table_build(float *cs, int T, int hd, float base, void *stream) {
    if (T < 0 || hd < 2 || hd > 256 || hd % 2 || !(base > 0.f)) return DTB_EINVAL_SHAPE;
    if (T == 0) return DTB_OK;
    if (!ptr_ok(cs)) return DTB_EINVAL_PTR;
    return rope_table(cs, T, hd, base, (hipStream_t)stream);
}

int block_saved_layout(const dtb_block_cfg *cfg, dtb_saved_layout *layout) {
    Dims d;
    int e = check_cfg(cfg, &d);
    if (e) return e;
    if (!layout) return DTB_EINVAL_PTR;
    saved_layout(cfg, d, layout);
    return DTB_OK;
}

size_t block_workspace_bytes(const dtb_block_cfg *cfg) {
    Dims d;
    if (check_cfg(cfg, &d)) return 0;
    WsLayout W;
    ws_layout(cfg, d, &W);
    return W.total;
}

int block_workspace_layout(const dtb_block_cfg *cfg, dtb_workspace_layout *layout) {
    Dims d;
    int e = check_cfg(cfg, &d);
    if (e) return e;
    if (!layout) return DTB_EINVAL_PTR;
    WsLayout W;
    ws_layout(cfg, d, &W);
    layout->dh = (long long)W.dh;
    layout->dup = (long long)W.dup;
    layout->dn2 = (long long)W.dn2;
    layout->dx2 = (long long)W.dx2;
    layout->dO = (long long)W.dO;
    layout->dqkv = (long long)W.dqkv;
    layout->dn1 = (long long)W.dn1;
    layout->total = (long long)W.total;
    return DTB_OK;
}

size_t attn_workspace_bytes(int B, int T, int NH) {
    if (B < 0 || T < 0 || NH <= 0) return 0;
    size_t n = (size_t)B * T * NH * 4 * 2;  // -D and -lse / scale
    return n ? al(n) : 256;
}

int attn_forward(void *out, float *lse, const void *qkv, int B, int T, int C, int NH, int NKV, int dtype,
                 void *stream) {
    int e = check_attn_shape(B, T, C, NH, NKV, dtype);
    if (e) return e;
    if ((long long)B * T == 0) return DTB_OK;
    if (!ptr_ok(out) || !ptr_ok(lse) || !ptr_ok(qkv)) return DTB_EINVAL_PTR;
    return launch_attn_forward(out, lse, qkv, B, T, C, NH, NKV, dtype, (hipStream_t)stream);
}

int attn_backward(void *dqkv, const void *qkv, const void *out, const void *dout, const float *lse, int B, int T,
                  int C, int NH, int NKV, int dtype, void *workspace, void *stream) {
    int e = check_attn_shape(B, T, C, NH, NKV, dtype);
    if (e) return e;
    if ((long long)B * T == 0) return DTB_OK;
    if (!ptr_ok(dqkv) || !ptr_ok(qkv) || !ptr_ok(out) || !ptr_ok(dout) || !ptr_ok(lse) || !ptr_ok(workspace))
        return DTB_EINVAL_PTR;
    return launch_attn_backward(dqkv, qkv, out, dout, lse, B, T, C, NH, NKV, dtype, (float *)workspace, nullptr,
                                (hipStream_t)stream);
}

// ---- attn_backward without a workspace argument ------------------------------
// The scratch of attn_backward_noalloc (-D and -lse / scale, [B][NH][T] fp32
// each) lives in this file-scope device array: every device the library runs
// on holds its own copy from module load until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, asked once per device with that device current, and
// is kept per device.
static __device__ __align__(256) char scratch[DTB_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
static void *g_scratch_ptr[kMaxDevices];

static int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_launch_error(e, "attn_backward_noalloc (hipGetDevice)");
    if (dev < 0 || dev >= kMaxDevices) return set_launch_error(hipErrorInvalidDevice, "attn_backward_noalloc");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return set_launch_error(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                             "attn_backward_noalloc (hipGetSymbolAddress)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DTB_OK;
}

int attn_backward_noalloc(void *dqkv, const void *qkv, const void *out, const void *dout, const float *lse, int B,
                          int T, int C, int NH, int NKV, int dtype, void *stream) {
    int e = check_attn_shape(B, T, C, NH, NKV, dtype);
    if (e) return e;
    if ((long long)B * T == 0) return DTB_OK;
    // -D and -lse / scale, each [B][NH][T] fp32, must fit the array
    if ((long long)B * NH * T * 4 * 2 > (long long)DTB_NOALLOC_SCRATCH_BYTES) return DTB_EINVAL_SHAPE;
    if (!ptr_ok(dqkv) || !ptr_ok(qkv) || !ptr_ok(out) || !ptr_ok(dout) || !ptr_ok(lse)) return DTB_EINVAL_PTR;
    void *ws = nullptr;
    e = scratch_address(&ws);
    if (e) return e;
    // the backward's kernels write every scratch value they read (nothing has
    // to start at zero), so no clearing pass is needed
    return launch_attn_backward(dqkv, qkv, out, dout, lse, B, T, C, NH, NKV, dtype, (float *)ws, nullptr,
                                (hipStream_t)stream);
}

static int check_decode(int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (B < 0 || Tmax < 0 || NH <= 0 || NKV <= 0 || NH % NKV || chunk < 0 || chunk % 32) return DTB_EINVAL_SHAPE;
    if (!hd_ok(hd, dtype)) return DTB_EINVAL_SHAPE;
    const long long es = dtype == DTB_BF16 ? 2 : 4;
    if ((long long)Tmax * NKV * hd * es >= (1LL << 31) || (long long)B * NH * hd >= (1LL << 31))
        return DTB_EINVAL_SHAPE;
    if ((long long)B * NKV * ((Tmax + 31) / 32) * NH >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

size_t attn_decode_workspace_bytes(int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype) {
    if (check_decode(B, NH, NKV, hd, Tmax, chunk, dtype)) return 0;
    size_t n = decode_geometry(B, NH, NKV, hd, Tmax, chunk, dtype).ws_bytes;
    return n ? al(n) : 256;
}

static int decode_run(void *out, float *lse, const void *q, const void *k_cache, const void *v_cache,
                      const int *lens, int B, int NH, int NKV, int hd, int Tmax, long long sb, long long st,
                      long long sh, int chunk, int dtype, void *workspace, void *stream) {
    if (B == 0) return DTB_OK;
    if (!ptr_ok(out) || !ptr_ok(lse) || !ptr_ok(q) || !ptr_ok(lens) || !ptr_ok(workspace)) return DTB_EINVAL_PTR;
    if (Tmax > 0 && (!ptr_ok(k_cache) || !ptr_ok(v_cache))) return DTB_EINVAL_PTR;
    const DecodeGeom g = decode_geometry(B, NH, NKV, hd, Tmax, chunk, dtype);
    hipError_t he = attn_decode_launch(out, lse, q, k_cache, v_cache, lens, B, NH, NKV, hd, Tmax, sb, st, sh, g,
                                       dtype, workspace, (hipStream_t)stream);
    if (he != hipSuccess) return set_launch_error(he, "attn_decode");
    return DTB_OK;
}

int attn_decode(void *out, float *lse, const void *q, const void *k_cache, const void *v_cache, const int *lens,
                int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype, void *workspace, void *stream) {
    int e = check_decode(B, NH, NKV, hd, Tmax, chunk, dtype);
    if (e) return e;
    const long long row = (long long)NKV * hd;
    return decode_run(out, lse, q, k_cache, v_cache, lens, B, NH, NKV, hd, Tmax, (long long)Tmax * row, row, hd,
                      chunk, dtype, workspace, stream);
}

int attn_decode_strided(void *out, float *lse, const void *q, const void *k_cache, const void *v_cache,
                        const int *lens, int B, int NH, int NKV, int hd, int Tmax, long long stride_b,
                        long long stride_t, long long stride_h, int chunk, int dtype, void *workspace,
                        void *stream) {
    int e = check_decode(B, NH, NKV, hd, Tmax, chunk, dtype);
    if (e) return e;
    const long long es = dtype == DTB_BF16 ? 2 : 4;
    // every head row lies inside its (b, kv head) base's 2^31-byte window, and
    // the rows of one sequence and kv head do not overlap
    if (stride_b < 0 || stride_t < hd || stride_h < 0) return DTB_EINVAL_SHAPE;
    if (Tmax > 0 && ((long long)(Tmax - 1) * stride_t + hd) * es >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    return decode_run(out, lse, q, k_cache, v_cache, lens, B, NH, NKV, hd, Tmax, stride_b, stride_t, stride_h,
                      chunk, dtype, workspace, stream);
}

static int check_linear(int R, int K, int N, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (R < 0 || K <= 0 || N <= 0 || K % 8 || N % 8) return DTB_EINVAL_SHAPE;
    if ((long long)R * (K > N ? K : N) >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

size_t linear_workspace_bytes(int R, int K, int N, int dtype) {
    if (check_linear(R, K, N, dtype)) return 0;
    size_t g = gemm_ws_bytes(N, K, R, dtype);
    size_t b = (size_t)bias_grad_parts(R) * N * 4;
    return al(g) + al(b) + 256;
}

int linear_forward(void *out, const void *inp, const void *w, const void *bias, const void *res, int R, int K,
                   int N, int dtype, void *stream) {
    int e = check_linear(R, K, N, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(out) || !ptr_ok(inp) || !ptr_ok(w)) return DTB_EINVAL_PTR;
    if ((bias && !aligned(bias)) || (res && !aligned(res))) return DTB_EINVAL_PTR;
    GemmArgs g{};
    g.dtype = dtype;
    g.a_kmajor = g.b_kmajor = true;
    g.A = inp; g.lda = K; g.B = w; g.ldb = K; g.M = R; g.N = N; g.K = K;
    g.out = out; g.ldo = N; g.bias = bias; g.res = res; g.ldr = N;
    return gemm(g, nullptr, 0, (hipStream_t)stream);
}

int linear_backward(void *dinp, float *dw, float *db, const void *dout, const void *inp, const void *w, int R,
                    int K, int N, int dtype, void *workspace, void *stream) {
    int e = check_linear(R, K, N, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(dout) || (dinp && !ptr_ok(w)) || (dw && !ptr_ok(inp))) return DTB_EINVAL_PTR;
    if ((dinp && !aligned(dinp)) || (dw && !aligned(dw)) || (db && !aligned(db))) return DTB_EINVAL_PTR;
    if ((dw || db) && !ptr_ok(workspace)) return DTB_EINVAL_PTR;
    hipStream_t s = (hipStream_t)stream;
    if (dinp) {
        GemmArgs g{};
        g.dtype = dtype;
        g.a_kmajor = true;
        g.b_kmajor = false;
        g.A = dout; g.lda = N; g.B = w; g.ldb = K; g.M = R; g.N = K; g.K = N; g.out = dinp; g.ldo = K;
        int r = gemm(g, nullptr, 0, s);
        if (r) return r;
    }
    size_t gbytes = gemm_ws_bytes(N, K, R, dtype);
    if (dw) {
        GemmArgs g{};
        g.dtype = dtype;
        g.a_kmajor = g.b_kmajor = false;
        g.out_f32 = g.accumulate = true;
        g.A = dout; g.lda = N; g.B = inp; g.ldb = K; g.M = N; g.N = K; g.K = R; g.out = dw; g.ldo = K;
        int r = gemm(g, workspace, gbytes, s);
        if (r) return r;
    }
    if (db) {
        float *part = (float *)((char *)workspace + al(gbytes));
        int r = bias_grad(dtype, dout, R, N, db, part, bias_grad_parts(R), s);
        if (r) return r;
    }
    return DTB_OK;
}

// ---- model harness -----------------------------------------------------------
static bool aligned4(const void *p) { return p && ((uintptr_t)p & 3) == 0; }

int encoder_forward(void *x, const int *ids, const void *wte, const void *wpe, int B, int T, int C, int V,
                    int dtype, void *stream) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (B < 0 || T < 0 || C <= 0 || C % 8 || V <= 0 || (long long)B * T >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    if ((long long)B * T == 0) return DTB_OK;
    if (!ptr_ok(x) || !aligned4(ids) || !ptr_ok(wte) || (wpe && !aligned(wpe))) return DTB_EINVAL_PTR;
    return embed_fwd(dtype, ids, wte, wpe, (long)B * T, T, C, V, x, (hipStream_t)stream);
}

int encoder_backward(float *dwte, float *dwpe, const int *ids, const void *dx, int B, int T, int C, int V,
                     int dtype, void *stream) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (B < 0 || T < 0 || C <= 0 || C % 8 || V <= 0 || (long long)B * T >= (1LL << 31)) return DTB_EINVAL_SHAPE;
    if ((long long)B * T == 0) return DTB_OK;
    if (!ptr_ok(dx) || (dwte && (!aligned(dwte) || !aligned4(ids))) || (dwpe && !aligned(dwpe)))
        return DTB_EINVAL_PTR;
    return embed_bwd(dtype, ids, dx, B, T, C, V, dwte, dwpe, (hipStream_t)stream);
}

static int check_norm(int R, int C, int norm, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (norm < 0 || norm > 2) return DTB_EINVAL_ENUM;
    if (R < 0 || C <= 0 || C % 8 || C > (dtype == DTB_BF16 ? 8192 : 4096)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

int norm_forward(void *out, float *rstd, float *mean, const void *x, const void *g, const void *b, int R, int C,
                 int norm, float eps, int dtype, void *stream) {
    int e = check_norm(R, C, norm, dtype);
    if (e) return e;
    if (!(eps > 0.f)) return DTB_EINVAL_SHAPE;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(out) || !ptr_ok(rstd) || !ptr_ok(x)) return DTB_EINVAL_PTR;
    if (norm != DTB_NORM_RMS_NOGAMMA && !ptr_ok(g)) return DTB_EINVAL_PTR;
    if (norm == DTB_NORM_LAYER && (!ptr_ok(b) || !ptr_ok(mean))) return DTB_EINVAL_PTR;
    return dtb::norm_forward(norm, dtype, x, g, b, eps, R, C, out, rstd, mean, (hipStream_t)stream);
}

size_t norm_workspace_bytes(int R, int C) {
    if (R < 0 || C <= 0) return 0;
    return al(norm_backward_ws_bytes(R, C));
}

int norm_backward(void *dx, float *dg, float *db, const void *dy, const void *x, const void *g, const float *rstd,
                  const float *mean, const void *dres, int R, int C, int norm, int dtype, void *workspace,
                  void *stream) {
    int e = check_norm(R, C, norm, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(dx) || !ptr_ok(dy) || !ptr_ok(x) || !ptr_ok(rstd) || !ptr_ok(workspace)) return DTB_EINVAL_PTR;
    if (dres && !aligned(dres)) return DTB_EINVAL_PTR;
    if (norm != DTB_NORM_RMS_NOGAMMA && (!ptr_ok(g) || !ptr_ok(dg))) return DTB_EINVAL_PTR;
    if (norm == DTB_NORM_LAYER && (!ptr_ok(db) || !ptr_ok(mean))) return DTB_EINVAL_PTR;
    return dtb::norm_backward(norm, dtype, dy, x, g, rstd, mean, dres, R, C, dx, dg, db, (float *)workspace,
                              norm_backward_parts(R), (hipStream_t)stream);
}

static int check_act(int R, int H, int mlp, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (mlp < 0 || mlp > 2) return DTB_EINVAL_ENUM;
    if (R < 0 || H <= 0 || H % 8 || (long long)R * H >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

int activation_forward(void *h, const void *up, int R, int H, int mlp, int dtype, void *stream) {
    int e = check_act(R, H, mlp, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(h) || !ptr_ok(up)) return DTB_EINVAL_PTR;
    return dtb::act_forward(mlp, dtype, up, R, H, h, (hipStream_t)stream);
}

int activation_backward(void *dup, const void *dh, const void *up, int R, int H, int mlp, int dtype, void *stream) {
    int e = check_act(R, H, mlp, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(dup) || !ptr_ok(dh) || !ptr_ok(up)) return DTB_EINVAL_PTR;
    return dtb::act_backward(mlp, dtype, dh, up, R, H, dup, (hipStream_t)stream);
}

static int check_head(int R, int C, int V, int ldl, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (R < 0 || C <= 0 || C % 8 || V <= 0 || ldl < V || ldl % 8) return DTB_EINVAL_SHAPE;
    if ((long long)R * ldl >= (1LL << 40) || (long long)V * C >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}

int lm_head_forward(void *logits, int ldl, const void *inp, const void *w, int R, int C, int V, int dtype,
                    void *stream) {
    int e = check_head(R, C, V, ldl, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(logits) || !ptr_ok(inp) || !ptr_ok(w)) return DTB_EINVAL_PTR;
    GemmArgs g{};
    g.dtype = dtype;
    g.a_kmajor = g.b_kmajor = true;
    g.A = inp; g.lda = C; g.B = w; g.ldb = C; g.M = R; g.N = V; g.K = C;
    g.out = logits; g.ldo = ldl;
    return gemm(g, nullptr, 0, (hipStream_t)stream);
}

size_t lm_head_workspace_bytes(int R, int C, int V, int dtype) {
    if (R < 0 || C <= 0 || V <= 0 || (dtype != DTB_F32 && dtype != DTB_BF16)) return 0;
    return al(gemm_ws_bytes(V, C, R, dtype)) + 256;
}

int lm_head_backward(void *dinp, float *dw, const void *dlogits, int ldl, const void *inp, const void *w, int R,
                     int C, int V, int dtype, void *workspace, void *stream) {
    int e = check_head(R, C, V, ldl, dtype);
    if (e) return e;
    if (R == 0) return DTB_OK;
    if (!ptr_ok(dlogits) || (dinp && (!ptr_ok(w) || !aligned(dinp))) || (dw && (!ptr_ok(inp) || !aligned(dw))))
        return DTB_EINVAL_PTR;
    if (dw && !ptr_ok(workspace)) return DTB_EINVAL_PTR;
    hipStream_t s = (hipStream_t)stream;
    if (dinp) {  // dinp[R, C] = dlogits[R, :V] W[V, C]
        GemmArgs g{};
        g.dtype = dtype;
        g.a_kmajor = true;
        g.b_kmajor = false;
        g.A = dlogits; g.lda = ldl; g.B = w; g.ldb = C; g.M = R; g.N = C; g.K = V; g.out = dinp; g.ldo = C;
        int r = gemm(g, nullptr, 0, s);
        if (r) return r;
    }
    if (dw) {  // dw[V, C] += dlogits[:, :V]^T inp
        GemmArgs g{};
        g.dtype = dtype;
        g.a_kmajor = g.b_kmajor = false;
        g.out_f32 = g.accumulate = true;
        g.A = dlogits; g.lda = ldl; g.B = inp; g.ldb = C; g.M = V; g.N = C; g.K = R; g.out = dw; g.ldo = C;
        int r = gemm(g, workspace, gemm_ws_bytes(V, C, R, dtype), s);
        if (r) return r;
    }
    return DTB_OK;
}

int softmax_ce(float *loss, float *row_loss, void *dlogits, const void *logits, int ldl, const int *targets, int R,
               int V, float scale, int dtype, void *stream) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (R < 0 || V <= 0 || ldl < V || ldl % 8 || (long long)R * ldl >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    if (!ptr_ok(loss) || (R > 0 && (!ptr_ok(row_loss) || !ptr_ok(dlogits) || !ptr_ok(logits) || !aligned4(targets))))
        return DTB_EINVAL_PTR;
    return softmax_xent_rows(dtype, logits, ldl, targets, R, V, scale, row_loss, dlogits, loss, (hipStream_t)stream);
}

static int check_head_ce(int R, int C, int V, int vchunk, int dtype) {
    if (dtype != DTB_F32 && dtype != DTB_BF16) return DTB_EDTYPE;
    if (R < 0 || C <= 0 || C % 8 || V <= 0 || vchunk < 0 || vchunk % 256) return DTB_EINVAL_SHAPE;
    if ((long long)R * C >= (1LL << 40) || (long long)V * C >= (1LL << 40)) return DTB_EINVAL_SHAPE;
    return DTB_OK;
}
static int head_chunk(int V, int vchunk) { return vchunk > 0 ? (vchunk < V ? vchunk : (V + 255) / 256 * 256) : (V < 4096 ? (V + 255) / 256 * 256 : 4096); }

size_t lm_head_ce_workspace_bytes(int R, int C, int V, int vchunk, int dtype) {
    if (check_head_ce(R, C, V, vchunk, dtype)) return 0;
    return head_ce_ws_bytes(R, C, V, head_chunk(V, vchunk), dtype);
}

int lm_head_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w, const int *targets,
               int R, int C, int V, int vchunk, float scale, int dtype, void *workspace, void *stream) {
    int e = check_head_ce(R, C, V, vchunk, dtype);
    if (e) return e;
    if (!ptr_ok(loss)) return DTB_EINVAL_PTR;
    if (R > 0 && (!ptr_ok(row_loss) || !ptr_ok(inp) || !ptr_ok(w) || !aligned4(targets) || !ptr_ok(workspace)))
        return DTB_EINVAL_PTR;
    if ((dinp && !aligned(dinp)) || (dw && !aligned(dw))) return DTB_EINVAL_PTR;
    return head_ce(loss, row_loss, dinp, dw, inp, w, targets, R, C, V, 1, head_chunk(V, vchunk), scale, dtype,
                   workspace, (hipStream_t)stream);
}

int lm_head_mtp_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w,
                   const int *targets, int R, int C, int V, int K, int vchunk, float scale, int dtype, void *workspace,
                   void *stream) {
    int e = check_head_ce(R, C, V, vchunk, dtype);
    if (e) return e;
    if (K < 1 || (long long)K * V >= (1LL << 31) || (long long)K * V * C >= (1LL << 40) ||
        (long long)R * K >= (1LL << 31))
        return DTB_EINVAL_SHAPE;
    if (!ptr_ok(loss)) return DTB_EINVAL_PTR;
    if (R > 0 && (!ptr_ok(row_loss) || !ptr_ok(inp) || !ptr_ok(w) || !aligned4(targets) || !ptr_ok(workspace)))
        return DTB_EINVAL_PTR;
    if ((dinp && !aligned(dinp)) || (dw && !aligned(dw))) return DTB_EINVAL_PTR;
    return head_ce(loss, row_loss, dinp, dw, inp, w, targets, R, C, V, K, head_chunk(V, vchunk), scale, dtype,
                   workspace, (hipStream_t)stream);
}

int adamw_update(float *params, float *grads, float *m, float *v, void *params_lowp, long long n, float lr,
                 float beta1, float beta2, float eps, float weight_decay, int step, int lowp_dtype, int zero_grads,
                 void *stream) {
    if (n < 0 || step < 1) return DTB_EINVAL_SHAPE;
    if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps >= 0.f)) return DTB_EINVAL_SHAPE;
    if (params_lowp && lowp_dtype != DTB_BF16) return DTB_EDTYPE;
    if (n == 0) return DTB_OK;
    if (!ptr_ok(params) || !ptr_ok(grads) || !ptr_ok(m) || !ptr_ok(v) || (params_lowp && !aligned(params_lowp)))
        return DTB_EINVAL_PTR;
    return adamw(params, grads, m, v, params_lowp, n, lr, beta1, beta2, eps, weight_decay, step, zero_grads,
                 (hipStream_t)stream);
}

static int check_weights(const dtb_block_cfg *c, const dtb_block_weights *w) {
    if (!w) return DTB_EINVAL_PTR;
    if (!ptr_ok(w->wqkv) || !ptr_ok(w->wo) || !ptr_ok(w->w_up) || !ptr_ok(w->w_down)) return DTB_EINVAL_PTR;
    if (c->norm != DTB_NORM_RMS_NOGAMMA && (!ptr_ok(w->g1) || !ptr_ok(w->g2))) return DTB_EINVAL_PTR;
    if (c->norm == DTB_NORM_LAYER && (!ptr_ok(w->b1) || !ptr_ok(w->b2))) return DTB_EINVAL_PTR;
    if (c->qkv_bias && !ptr_ok(w->bqkv)) return DTB_EINVAL_PTR;
    if (c->o_bias && !ptr_ok(w->bo)) return DTB_EINVAL_PTR;
    if (c->mlp_bias && (!ptr_ok(w->b_up) || !ptr_ok(w->b_down))) return DTB_EINVAL_PTR;
    if (w->rope_cs && !aligned(w->rope_cs)) return DTB_EINVAL_PTR;
    return DTB_OK;
}

static int check_grads(const dtb_block_cfg *c, const dtb_block_grads *g) {
    if (!g) return DTB_EINVAL_PTR;
    if (!ptr_ok(g->wqkv) || !ptr_ok(g->wo) || !ptr_ok(g->w_up) || !ptr_ok(g->w_down)) return DTB_EINVAL_PTR;
    if (c->norm != DTB_NORM_RMS_NOGAMMA && (!ptr_ok(g->g1) || !ptr_ok(g->g2))) return DTB_EINVAL_PTR;
    if (c->norm == DTB_NORM_LAYER && (!ptr_ok(g->b1) || !ptr_ok(g->b2))) return DTB_EINVAL_PTR;
    if (c->qkv_bias && !ptr_ok(g->bqkv)) return DTB_EINVAL_PTR;
    if (c->o_bias && !ptr_ok(g->bo)) return DTB_EINVAL_PTR;
    if (c->mlp_bias && (!ptr_ok(g->b_up) || !ptr_ok(g->b_down))) return DTB_EINVAL_PTR;
    return DTB_OK;
}

#define TRY(x)                  \
    do {                        \
        int _r = (x);           \
        if (_r) return _r;      \
    } while (0)

int block_forward(const dtb_block_cfg *c, const dtb_block_weights *w, const void *x_in, void *x_out, void *saved,
                  void *workspace, void *stream) {
    Dims d;
    TRY(check_cfg(c, &d));
    if (d.BT == 0) return DTB_OK;
    TRY(check_weights(c, w));
    if (!ptr_ok(x_in) || !ptr_ok(x_out) || !ptr_ok(saved) || !ptr_ok(workspace)) return DTB_EINVAL_PTR;
    hipStream_t s = (hipStream_t)stream;
    dtb_saved_layout L;
    saved_layout(c, d, &L);
    WsLayout W;
    ws_layout(c, d, &W);
    char *sv = (char *)saved, *ws = (char *)workspace;
    const int C = c->C, H = c->H, BT = (int)d.BT, dt = c->dtype;
    void *n1 = sv + L.n1, *qkv = sv + L.qkv, *o = sv + L.o, *x2 = sv + L.x2, *n2 = sv + L.n2, *up = sv + L.up,
         *h = sv + L.h;
    float *r1 = (float *)(sv + L.r1), *r2 = (float *)(sv + L.r2);
    float *mu1 = L.mu1 >= 0 ? (float *)(sv + L.mu1) : nullptr, *mu2 = L.mu2 >= 0 ? (float *)(sv + L.mu2) : nullptr;
    float *lse = (float *)(sv + L.lse);

    TRY(norm_forward(c->norm, dt, x_in, w->g1, w->b1, c->eps, BT, C, n1, r1, mu1, s));
    GemmArgs g{};
    g.dtype = dt;
    g.a_kmajor = g.b_kmajor = true;
    // qkv = RoPE(n1 Wqkv^T + bqkv) on the q and k heads (rotation in the GEMM epilogue)
    g.A = n1; g.lda = C; g.B = w->wqkv; g.ldb = C; g.M = BT; g.N = d.QKV; g.K = C;
    g.out = qkv; g.ldo = d.QKV; g.bias = c->qkv_bias ? w->bqkv : nullptr; g.res = nullptr;
    if (c->rope == DTB_ROPE_NEOX) {
        const float *cs = w->rope_cs;
        if (!cs) {
            TRY(rope_table((float *)(ws + W.cs), c->T, d.hd, c->rope_base, s));
            cs = (const float *)(ws + W.cs);
        }
        g.rope_cs = cs; g.rope_T = c->T; g.rope_hd = d.hd; g.rope_cols = C + c->NKV * d.hd;
    }
    TRY(gemm(g, nullptr, 0, s));
    g.rope_cs = nullptr;
    TRY(launch_attn_forward(o, lse, qkv, c->B, c->T, C, c->NH, c->NKV, dt, s));
    // x2 = x + o Wo^T + bo
    g.A = o; g.lda = C; g.B = w->wo; g.ldb = C; g.M = BT; g.N = C; g.K = C;
    g.out = x2; g.ldo = C; g.bias = c->o_bias ? w->bo : nullptr; g.res = x_in; g.ldr = C;
    TRY(gemm(g, nullptr, 0, s));
    TRY(norm_forward(c->norm, dt, x2, w->g2, w->b2, c->eps, BT, C, n2, r2, mu2, s));
    // up = n2 Wup^T + bup; h = activation(up) (in the GEMM epilogue where the tiling allows)
    g.A = n2; g.lda = C; g.B = w->w_up; g.ldb = C; g.M = BT; g.N = d.W; g.K = C;
    g.out = up; g.ldo = d.W; g.bias = c->mlp_bias ? w->b_up : nullptr; g.res = nullptr;
    g.act_h = h; g.act_mode = c->mlp; g.act_H = H;
    TRY(gemm(g, nullptr, 0, s));
    g.act_h = nullptr;
    // x_out = x2 + h Wdown^T + bdown
    g.A = h; g.lda = H; g.B = w->w_down; g.ldb = H; g.M = BT; g.N = C; g.K = H;
    g.out = x_out; g.ldo = C; g.bias = c->mlp_bias ? w->b_down : nullptr; g.res = x2; g.ldr = C;
    TRY(gemm(g, nullptr, 0, s));
    return DTB_OK;
}

int dtb_overlap_create(dtb_overlap *out) {
    if (!out) return DTB_EINVAL_PTR;
    *out = nullptr;
    dtb_overlap h = new (std::nothrow) dtb_overlap_s{};
    if (!h) return set_launch_error(hipErrorOutOfMemory, "dtb_overlap_create");
    hipError_t e = hipGetDevice(&h->device);
    // default priority (a stream of another priority is never created)
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)dtb_overlap_destroy(h);
        return set_launch_error(e, "dtb_overlap_create");
    }
    *out = h;
    return DTB_OK;
}

int dtb_overlap_destroy(dtb_overlap h) {
    if (!h) return DTB_OK;
    // no wait: HIP releases a stream or an event with pending work once that
    // work has completed
    if (h->join) (void)hipEventDestroy(h->join);
    if (h->fork) (void)hipEventDestroy(h->fork);
    if (h->s) (void)hipStreamDestroy(h->s);
    delete h;
    return DTB_OK;
}

static int block_backward_impl(const dtb_block_cfg *c, const dtb_block_weights *w, const void *x_in,
                               const void *saved, const void *dx_out, void *dx_in, const dtb_block_grads *gr,
                               void *workspace, void *stream, dtb_overlap side_h);

int block_backward(const dtb_block_cfg *c, const dtb_block_weights *w, const void *x_in, const void *saved,
                   const void *dx_out, void *dx_in, const dtb_block_grads *gr, void *workspace, void *stream) {
    return block_backward_impl(c, w, x_in, saved, dx_out, dx_in, gr, workspace, stream, nullptr);
}

int block_backward_overlap(const dtb_block_cfg *c, const dtb_block_weights *w, const void *x_in, const void *saved,
                           const void *dx_out, void *dx_in, const dtb_block_grads *gr, void *workspace, void *stream,
                           dtb_overlap side) {
    if (!side) return DTB_EINVAL_PTR;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != side->device) return DTB_EINVAL_PTR;
    return block_backward_impl(c, w, x_in, saved, dx_out, dx_in, gr, workspace, stream, side);
}

static int block_backward_impl(const dtb_block_cfg *c, const dtb_block_weights *w, const void *x_in,
                               const void *saved, const void *dx_out, void *dx_in, const dtb_block_grads *gr,
                               void *workspace, void *stream, dtb_overlap side_h) {
    Dims d;
    TRY(check_cfg(c, &d));
    if (d.BT == 0) return DTB_OK;
    TRY(check_weights(c, w));
    TRY(check_grads(c, gr));
    if (!ptr_ok(x_in) || !ptr_ok(saved) || !ptr_ok(dx_out) || !ptr_ok(dx_in) || !ptr_ok(workspace))
        return DTB_EINVAL_PTR;
    hipStream_t s = (hipStream_t)stream;
    dtb_saved_layout L;
    saved_layout(c, d, &L);
    WsLayout W;
    ws_layout(c, d, &W);
    const char *sv = (const char *)saved;
    char *ws = (char *)workspace;
    const int C = c->C, H = c->H, BT = (int)d.BT, dt = c->dtype;
    const void *n1 = sv + L.n1, *qkv = sv + L.qkv, *o = sv + L.o, *x2 = sv + L.x2, *n2 = sv + L.n2,
               *up = sv + L.up, *h = sv + L.h;
    const float *r1 = (const float *)(sv + L.r1), *r2 = (const float *)(sv + L.r2);
    const float *mu1 = L.mu1 >= 0 ? (const float *)(sv + L.mu1) : nullptr;
    const float *mu2 = L.mu2 >= 0 ? (const float *)(sv + L.mu2) : nullptr;
    const float *lse = (const float *)(sv + L.lse);
    void *dh = ws + W.dh, *dup = ws + W.dup, *dn2 = ws + W.dn2, *dx2 = ws + W.dx2, *dO = ws + W.dO,
         *dqkv = ws + W.dqkv, *dn1 = ws + W.dn1;
    float *Dbuf = (float *)(ws + W.D), *npart = (float *)(ws + W.npart), *bpart = (float *)(ws + W.bpart);
    void *gws = ws + W.gemm;
    const void *dy = dx_out;

    GemmArgs dinp{};
    dinp.dtype = dt;
    dinp.a_kmajor = true;
    dinp.b_kmajor = false;
    GemmArgs dw{};
    dw.dtype = dt;
    dw.a_kmajor = false;
    dw.b_kmajor = false;
    dw.out_f32 = true;
    dw.accumulate = true;

    // weight gradients on the side stream: each forks after the main stream
    // has produced its inputs and reads only buffers that nothing later in
    // this call writes, except dy, which the last kernel may overwrite (dx_in
    // may be dx_out): the main stream joins before that kernel
    dtb_overlap side = timing_serializes_backward() ? nullptr : side_h;
    hipStream_t s2 = side ? side->s : s;
    bool forked = false;
    auto fork = [&]() -> int {
        if (!side) return DTB_OK;
        forked = true;
        hipError_t e = hipEventRecord(side->fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(s2, side->fork, 0);
        return e == hipSuccess ? DTB_OK : set_launch_error(e, "block_backward fork");
    };
    auto join = [&]() -> int {
        if (!side || !forked) return DTB_OK;
        forked = false;
        hipError_t e = hipEventRecord(side->join, s2);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
        return e == hipSuccess ? DTB_OK : set_launch_error(e, "block_backward join");
    };
    // an early return (a launch error) still leaves the caller's stream
    // waiting for everything already enqueued on the side stream
    struct JoinOnExit {
        decltype(join) &j;
        ~JoinOnExit() { (void)j(); }
    } join_on_exit{join};

    // down projection: dh = dy Wdown; dWdown += dy^T h; db_down
    // (the activation backward stays a kernel of its own: in the GEMM epilogue
    // its 8 bytes per element of extra HBM traffic, which no MFMA work hides,
    // measured slower than the separate streaming pass)
    dinp.A = dy; dinp.lda = C; dinp.B = w->w_down; dinp.ldb = H; dinp.M = BT; dinp.N = H; dinp.K = C;
    dinp.out = dh; dinp.ldo = H;
    TRY(fork());
    TRY(gemm(dinp, nullptr, 0, s));
    dw.A = dy; dw.lda = C; dw.B = h; dw.ldb = H; dw.M = C; dw.N = H; dw.K = BT; dw.out = gr->w_down; dw.ldo = H;
    TRY(gemm(dw, gws, W.gemm_bytes, s2));
    if (c->mlp_bias) TRY(bias_grad(dt, dy, BT, C, gr->b_down, bpart, W.bparts, s));
    TRY(act_backward(c->mlp, dt, dh, up, BT, H, dup, s));
    // up projection: dn2 = dup Wup; dWup += dup^T n2
    dinp.A = dup; dinp.lda = d.W; dinp.B = w->w_up; dinp.ldb = C; dinp.M = BT; dinp.N = C; dinp.K = d.W;
    dinp.out = dn2; dinp.ldo = C;
    TRY(fork());
    TRY(gemm(dinp, nullptr, 0, s));
    dw.A = dup; dw.lda = d.W; dw.B = n2; dw.ldb = C; dw.M = d.W; dw.N = C; dw.K = BT; dw.out = gr->w_up; dw.ldo = C;
    TRY(gemm(dw, gws, W.gemm_bytes, s2));
    if (c->mlp_bias) TRY(bias_grad(dt, dup, BT, d.W, gr->b_up, bpart, W.bparts, s));
    // norm2 backward + residual: dx2 = dy + Norm2^T(dn2)
    TRY(norm_backward(c->norm, dt, dn2, x2, w->g2, r2, mu2, dy, BT, C, dx2, gr->g2, gr->b2, npart, W.nparts, s));
    // output projection: dO = dx2 Wo; dWo += dx2^T o
    dinp.A = dx2; dinp.lda = C; dinp.B = w->wo; dinp.ldb = C; dinp.M = BT; dinp.N = C; dinp.K = C;
    dinp.out = dO; dinp.ldo = C;
    TRY(fork());
    TRY(gemm(dinp, nullptr, 0, s));
    dw.A = dx2; dw.lda = C; dw.B = o; dw.ldb = C; dw.M = C; dw.N = C; dw.K = BT; dw.out = gr->wo; dw.ldo = C;
    TRY(gemm(dw, gws, W.gemm_bytes, s2));
    if (c->o_bias) TRY(bias_grad(dt, dx2, BT, C, gr->bo, bpart, W.bparts, s));
    // attention (dq and dk leave the kernels already rotated back by the transposed RoPE)
    const float *cs = nullptr;
    if (c->rope == DTB_ROPE_NEOX) {
        cs = w->rope_cs;
        if (!cs) {
            TRY(rope_table((float *)(ws + W.cs), c->T, d.hd, c->rope_base, s));
            cs = (const float *)(ws + W.cs);
        }
    }
    TRY(launch_attn_backward(dqkv, qkv, o, dO, lse, c->B, c->T, C, c->NH, c->NKV, dt, Dbuf, cs, s));
    // qkv projection: dn1 = dqkv Wqkv; dWqkv += dqkv^T n1
    dinp.A = dqkv; dinp.lda = d.QKV; dinp.B = w->wqkv; dinp.ldb = C; dinp.M = BT; dinp.N = C; dinp.K = d.QKV;
    dinp.out = dn1; dinp.ldo = C;
    TRY(fork());
    TRY(gemm(dinp, nullptr, 0, s));
    dw.A = dqkv; dw.lda = d.QKV; dw.B = n1; dw.ldb = C; dw.M = d.QKV; dw.N = C; dw.K = BT; dw.out = gr->wqkv;
    dw.ldo = C;
    TRY(gemm(dw, gws, W.gemm_bytes, s2));
    if (c->qkv_bias) TRY(bias_grad(dt, dqkv, BT, d.QKV, gr->bqkv, bpart, W.bparts, s));
    // norm1 backward + residual: dx_in = dx2 + Norm1^T(dn1); every weight
    // gradient has finished first (dx_in may be dy)
    TRY(join());
    TRY(norm_backward(c->norm, dt, dn1, x_in, w->g1, r1, mu1, dx2, BT, C, dx_in, gr->g1, gr->b1, npart, W.nparts,
                      s));
    return DTB_OK;
}

}  // extern "C"
