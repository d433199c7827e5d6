// fa_api.hip -- the C ABI declared in include/fa.h: argument checks (all on
// the host, before any HIP call), dispatch to the kernels, the decode
// workspace cache, and error reporting.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "fa.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace {

constexpr int kMaxSplits = 1024;
constexpr double kLog2e = 1.4426950408889634073599;

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int ok() {
    g_last_error.clear();
    return FA_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t element_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Any finite scale whose product with log2(e) is a finite float32 (the
// kernels work in base 2); negative and zero scales included.
bool scale_ok(float scale) {
    return std::isfinite(scale) && std::isfinite((float)((double)scale * kLog2e));
}
constexpr const char *kScaleMsg = "scale must be finite, with |scale| * log2(e) within float32 range";

// Checks shared by every forward entry point.  Returns FA_OK or the status
// to return, with the message set.
int check_common(const void *q, const void *k, const void *v, const void *out, const float *lse, int B, int H,
                 int Nq, int Nk, int d, float scale, int dtype) {
    if (!q || !k || !v || !out) return fail(FA_ERR_INVALID_ARG, "q, k, v and out must be non-null");
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
        return fail(FA_ERR_INVALID_ARG, "B, H, Nq, Nk and d must all be >= 1");
    if (!scale_ok(scale)) return fail(FA_ERR_INVALID_ARG, kScaleMsg);
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
        return fail(FA_ERR_UNSUPPORTED, "dtype must be FA_F32 (0), FA_F16 (1) or FA_BF16 (2)");
    if (d != 32 && d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 32, 64 or 128");
    if ((int64_t)B * H > INT32_MAX || (int64_t)Nq * d > INT32_MAX || (int64_t)Nk * d > INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "B*H, Nq*d and Nk*d must each fit in 31 bits");
    // every byte count below (tensors, split workspaces of up to 1024 chunks)
    // then stays far inside 64 bits; 2^48 elements is beyond any device
    if ((int64_t)B * H * ((int64_t)(Nq > Nk ? Nq : Nk) * d) > ((int64_t)1 << 48))
        return fail(FA_ERR_UNSUPPORTED, "B*H*N*d must not exceed 2^48 elements");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(FA_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(FA_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
    const size_t es = element_size(dtype);
    const size_t bh = (size_t)B * H;
    const size_t q_bytes = bh * Nq * d * es, kv_bytes = bh * Nk * d * es;
    const size_t lse_bytes = bh * Nq * sizeof(float);
    if (overlaps(out, q_bytes, q, q_bytes) || overlaps(out, q_bytes, k, kv_bytes) ||
        overlaps(out, q_bytes, v, kv_bytes))
        return fail(FA_ERR_INVALID_ARG, "out overlaps q, k or v");
    if (lse && (overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
                overlaps(lse, lse_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, out, q_bytes)))
        return fail(FA_ERR_INVALID_ARG, "lse overlaps q, k, v or out");
    return FA_OK;
}

int hip_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return ok();
    return fail(FA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
}

size_t workspace_bytes(int B, int H, int Nq, int d, int S) {
    const size_t floats = (size_t)B * H * Nq * S * ((size_t)d + 1);
    return (floats * sizeof(float) + 255) / 256 * 256;
}

// Prefill tile shape forced by FA_PREFILL_SHAPE (0 .. kNumPrefillShapes - 1,
// for sweeps), or -1.
int env_shape() {
    const char *env = std::getenv("FA_PREFILL_SHAPE");
    if (env && env[0] >= '0' && env[0] < '0' + fa::kNumPrefillShapes && env[1] == '\0') return env[0] - '0';
    return -1;
}

bool key_split_shape(int shape) { return shape == fa::kShapeW4Q32K2 || shape == fa::kShapeW4Q32K4; }

// The shape of full-grid, split and variable-length launches: the forced
// one unless it is a key-split shape, else the measured best for the head
// dim -- 32-key tiles at three waves per SIMD for d = 128, 64-key tiles at
// two waves per SIMD below.
int prefill_shape(int d) {
    const int e = env_shape();
    if (e >= 0 && !key_split_shape(e)) return e;
    return d >= 128 ? fa::kShapeW4Q32B32 : fa::kShapeW4Q32;
}

// Library-owned split workspaces (decode, and split prefill), one per
// (device, stream).  A workspace that must grow is replaced, never freed in
// place: work enqueued earlier (by this or another thread, or a captured
// graph) may still use the old buffer, so it is retired and freed only by
// fa_release_workspace.  Growth is geometric, so the retired buffers of a
// stream together are smaller than its live one.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void *>> g_retired;  // (device, buffer)

int get_workspace(size_t need, hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_status(err, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[std::make_pair(dev, stream)];
    if (w.bytes < need) {
        size_t bytes = w.bytes > need / 2 ? 2 * w.bytes : need;
        void *p = nullptr;
        err = hipMalloc(&p, bytes);
        if (err != hipSuccess && bytes > need) {  // the doubled size did not fit: take what is needed
            (void)hipGetLastError();              // clear the failed allocation's error
            bytes = need;
            err = hipMalloc(&p, bytes);
        }
        if (err != hipSuccess) {
            (void)hipGetLastError();
            return hip_status(err, "hipMalloc(workspace)");
        }
        if (w.ptr) g_retired.emplace_back(dev, w.ptr);
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return FA_OK;
}

int run_splitkv(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int Nk, int d,
                float scale, int S, void *ws, int dtype, hipStream_t stream) {
    const float sl = (float)((double)scale * kLog2e);
    return hip_status(fa::launch_splitkv(dtype, d, q, k, v, out, lse, B * H, Nk, sl, S, ws, stream),
                      "split-KV launch");
}

// Where fa_fwd's split workspace comes from: the library's cache (hipMalloc
// on first use per stream), or the static scratch array of fa_fwd_noalloc.
enum class WsSource { kCache, kScratch };

// Scratch of fa_fwd_noalloc: a file-scope device array, so the code object
// loader places one copy on every GPU the library runs on, held until the
// process ends.  In host code ``scratch`` names a host-side stand-in, not
// device memory: host code uses only the address hipGetSymbolAddress gives
// for the current device (kept per device below).  The split workspace
// needs no clearing (every chunk slot is written before the combine reads
// it), and calls that overlap on one GPU share the array and race.
constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of each device's copy, or null before first use

int get_scratch(size_t need, void **out) {
    if (need > kScratchBytes)  // also checked by the caller before any HIP call
        return fail(FA_ERR_WORKSPACE, "fa_fwd_noalloc: the call needs " + std::to_string(need) +
                                          " bytes of scratch, more than its " + std::to_string(kScratchBytes));
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_status(err, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "fa_fwd_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {  // first call on this device (it is current): find its copy
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return hip_status(err != hipSuccess ? err : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

// The largest chunk count whose split workspace (B*H*Nq rows of S*(d + 1)
// float32) fits in the scratch array.
int scratch_max_splits(int B, int H, int Nq, int d) {
    const size_t per_split = (size_t)B * H * Nq * ((size_t)d + 1) * sizeof(float);
    const size_t s = kScratchBytes / per_split;
    return s > (size_t)kMaxSplits ? kMaxSplits : (int)s;
}

// fa_fwd and fa_fwd_noalloc: checks, then dispatch (see fa.h).  With the
// scratch source a split that would not fit the scratch array takes fewer
// chunks (as many as fit); a prefill then runs unsplit if fewer than two
// fit, and a decode that cannot fit one chunk is rejected before any HIP
// call.
int forward(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int Nq, int Nk,
            int d, float scale, int causal, int dtype, hipStream_t stream, WsSource src) {
    int st = check_common(q, k, v, out, lse, B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    const bool scratch_src = src == WsSource::kScratch;
    auto take = [&](size_t need, void **ws) {
        return scratch_src ? get_scratch(need, ws) : get_workspace(need, stream, ws);
    };

    if (Nq == 1 && !causal && dtype != FA_F32) {
        int S = fa_default_num_splits(Nk);
        if (scratch_src) {
            const int fit = scratch_max_splits(B, H, 1, d);
            if (fit < 1)
                return fail(FA_ERR_WORKSPACE, "fa_fwd_noalloc: B*H*(d + 1)*4 = " +
                                                  std::to_string(workspace_bytes(B, H, 1, d, 1)) +
                                                  " bytes exceed its scratch of " + std::to_string(kScratchBytes));
            S = S < fit ? S : fit;
        }
        void *ws = nullptr;
        st = take(workspace_bytes(B, H, 1, d, S), &ws);
        if (st != FA_OK) return st;
        return run_splitkv(q, k, v, out, lse, B, H, Nk, d, scale, S, ws, dtype, stream);
    }
    const float sl = (float)((double)scale * kLog2e);
    if (dtype == FA_F32) {  // a grid too small for the GPU splits its key range, then combines
        int S = fa::f32_split_count(causal == 1, B * H, Nq, Nk);
        if (S > 1 && scratch_src) {
            const int fit = scratch_max_splits(B, H, Nq, d);
            if (fit < S) S = fit >= 2 ? fa::f32_split_normalise(causal == 1, Nq, Nk, fit) : 1;
        }
        void *ws = nullptr;
        if (S > 1) {
            st = take(workspace_bytes(B, H, Nq, d, S), &ws);
            if (st != FA_OK) return st;
        }
        return hip_status(
            fa::launch_prefill_f32(d, causal == 1, q, k, v, out, lse, B * H, Nq, Nk, sl, S, ws, stream),
            "fp32 prefill launch");
    }
    int shape = prefill_shape(d);
    int S = fa::prefill_split_count(d, causal == 1, shape, B * H, Nq, Nk);
    if (S > 1 && scratch_src) {
        const int fit = scratch_max_splits(B, H, Nq, d);
        if (fit < S) S = fit >= 2 ? fa::prefill_split_normalise(d, causal == 1, shape, Nq, Nk, fit) : 1;
    }
    if (S > 1) {  // a grid too small for the GPU: split the key range, then combine
        void *ws = nullptr;
        st = take(workspace_bytes(B, H, Nq, d, S), &ws);
        if (st != FA_OK) return st;
        return hip_status(fa::launch_prefill_split(dtype, d, causal == 1, shape, q, k, v, out, lse, B * H, Nq, Nk,
                                                   sl, S, ws, stream),
                          "split prefill launch");
    }
    // a grid below one workgroup per CU: the key loop split over the waves of a workgroup
    shape = env_shape() >= 0 ? env_shape() : fa::prefill_small_grid_shape(d, causal == 1, shape, B * H, Nq, Nk);
    return hip_status(fa::launch_prefill(dtype, d, causal == 1, shape, q, k, v, out, lse, B * H, Nq, Nk, sl, stream),
                      "prefill launch");
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int Nq, int Nk, int d,
           float scale, int causal, int dtype, hipStream_t stream) {
    return forward(q, k, v, out, lse, B, H, Nq, Nk, d, scale, causal, dtype, stream, WsSource::kCache);
}

int fa_fwd_noalloc(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, int dtype, hipStream_t stream) {
    return forward(q, k, v, out, lse, B, H, Nq, Nk, d, scale, causal, dtype, stream, WsSource::kScratch);
}

size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits) {
    if (B < 1 || H < 1 || Nq < 1 || d < 1 || num_splits < 1 || num_splits > kMaxSplits) return 0;
    return workspace_bytes(B, H, Nq, d, num_splits);
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H, int Nq, int Nk,
                   int d, float scale, int num_splits, void *workspace, size_t ws_bytes, int dtype,
                   hipStream_t stream) {
    int st = check_common(q, k, v, out, lse, B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FA_ERR_INVALID_ARG, "num_splits must be in [1, 1024]");
    if (Nq != 1) return fail(FA_ERR_UNSUPPORTED, "the split-KV path takes Nq == 1 (single-token decode)");
    if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the split-KV path takes fp16 or bf16");
    const size_t need = workspace_bytes(B, H, Nq, d, num_splits);
    if (!workspace || !aligned(workspace, 16) || ws_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold fa_splitkv_workspace_bytes() = " +
                                          std::to_string(need) + " bytes");
    const size_t es = element_size(dtype);
    const size_t bh = (size_t)B * H;
    if (overlaps(workspace, need, q, bh * d * es) || overlaps(workspace, need, k, bh * Nk * d * es) ||
        overlaps(workspace, need, v, bh * Nk * d * es) || overlaps(workspace, need, out, bh * d * es) ||
        (lse && overlaps(workspace, need, lse, bh * sizeof(float))))
        return fail(FA_ERR_WORKSPACE, "workspace overlaps an input or output");
    return run_splitkv(q, k, v, out, lse, B, H, Nk, d, scale, num_splits, workspace, dtype, stream);
}

int fa_fwd_paged_decode(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                        const int *seq_lens, void *out, float *lse, int B, int H, int d, int block_size,
                        int max_blocks, int num_blocks, float scale, int num_splits, void *workspace,
                        size_t ws_bytes, int dtype, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
        return fail(FA_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, seq_lens and out must be non-null");
    if (B < 1 || H < 1 || d < 1 || block_size < 1 || max_blocks < 1 || num_blocks < 1)
        return fail(FA_ERR_INVALID_ARG, "B, H, d, block_size, max_blocks_per_seq and num_blocks must be >= 1");
    if (!scale_ok(scale)) return fail(FA_ERR_INVALID_ARG, kScaleMsg);
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FA_ERR_INVALID_ARG, "num_splits must be in [1, 1024]");
    if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the paged path takes fp16 or bf16");
    if (d != 32 && d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 32, 64 or 128");
    if (block_size > 1024 || (block_size & (block_size - 1)) != 0)
        return fail(FA_ERR_UNSUPPORTED, "block_size must be a power of two in [1, 1024]");
    if ((int64_t)B * H > INT32_MAX || (int64_t)max_blocks * block_size > INT32_MAX ||
        (int64_t)B * max_blocks > INT32_MAX || (int64_t)num_blocks * H > INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "B*H, max_blocks_per_seq*block_size, B*max_blocks_per_seq and "
                                         "num_blocks*H must each fit in 31 bits");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(FA_ERR_UNSUPPORTED, "q, k_cache, v_cache and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(FA_ERR_UNSUPPORTED, "block_table, seq_lens and lse must be 4-byte aligned");
    const size_t es = element_size(dtype);
    const size_t bh = (size_t)B * H;
    const size_t q_bytes = bh * d * es, cache_bytes = (size_t)num_blocks * H * block_size * d * es;
    const size_t table_bytes = (size_t)B * max_blocks * 4, lens_bytes = (size_t)B * 4, lse_bytes = bh * 4;
    const void *ins[5] = {q, k_cache, v_cache, block_table, seq_lens};
    const size_t in_bytes[5] = {q_bytes, cache_bytes, cache_bytes, table_bytes, lens_bytes};
    for (int i = 0; i < 5; ++i) {
        if (overlaps(out, q_bytes, ins[i], in_bytes[i])) return fail(FA_ERR_INVALID_ARG, "out overlaps an input");
        if (lse && overlaps(lse, lse_bytes, ins[i], in_bytes[i]))
            return fail(FA_ERR_INVALID_ARG, "lse overlaps an input");
    }
    if (lse && overlaps(lse, lse_bytes, out, q_bytes)) return fail(FA_ERR_INVALID_ARG, "lse overlaps out");
    const size_t need = workspace_bytes(B, H, 1, d, num_splits);
    if (!workspace || !aligned(workspace, 16) || ws_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold fa_splitkv_workspace_bytes() = " +
                                          std::to_string(need) + " bytes");
    for (int i = 0; i < 5; ++i)
        if (overlaps(workspace, need, ins[i], in_bytes[i]))
            return fail(FA_ERR_WORKSPACE, "workspace overlaps an input");
    if (overlaps(workspace, need, out, q_bytes) || (lse && overlaps(workspace, need, lse, lse_bytes)))
        return fail(FA_ERR_WORKSPACE, "workspace overlaps an output");
    int log2_block = 0;
    while ((1 << log2_block) < block_size) ++log2_block;
    const float sl = (float)((double)scale * kLog2e);
    return hip_status(fa::launch_paged_decode(dtype, d, q, k_cache, v_cache, block_table, seq_lens, out, lse, B, H,
                                              log2_block, max_blocks, num_blocks, sl, num_splits, workspace, stream),
                      "paged decode launch");
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq, int d) {
    if (B < 1 || H < 1 || Nq < 1 || (d != 32 && d != 64 && d != 128)) return 0;
    if ((int64_t)B * H > INT32_MAX) return 0;
    return (fa::bwd_stats_bytes(B * H, Nq) + 255) / 256 * 256;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout, const float *lse,
           void *dq, void *dk, void *dv, int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
           void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!dout || !lse || !dq || !dk || !dv)
        return fail(FA_ERR_INVALID_ARG, "dout, lse, dq, dk and dv must be non-null");
    int st = check_common(q, k, v, out, nullptr, B, H, Nq, Nk, d, scale, dtype);
    if (st != FA_OK) return st;
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "the backward takes fp16 or bf16");
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
        return fail(FA_ERR_UNSUPPORTED, "dout, dq, dk and dv must be 16-byte aligned");
    if (!aligned(lse, 4)) return fail(FA_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
    const size_t need = fa_bwd_workspace_bytes(B, H, Nq, d);
    if (need == 0 || need > (size_t)INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "B*H*Nq is too large for the backward's statistics");
    const size_t es = element_size(dtype);
    const size_t bh = (size_t)B * H;
    const size_t q_bytes = bh * Nq * d * es, kv_bytes = bh * Nk * d * es, lse_bytes = bh * Nq * 4;
    const void *ins[6] = {q, k, v, out, dout, lse};
    const size_t in_bytes[6] = {q_bytes, kv_bytes, kv_bytes, q_bytes, q_bytes, lse_bytes};
    void *outs[3] = {dq, dk, dv};
    const size_t out_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[o], out_bytes[o], ins[i], in_bytes[i]))
                return fail(FA_ERR_INVALID_ARG, "dq, dk and dv must not overlap an input");
        for (int p = 0; p < o; ++p)
            if (overlaps(outs[o], out_bytes[o], outs[p], out_bytes[p]))
                return fail(FA_ERR_INVALID_ARG, "dq, dk and dv must not overlap each other");
    }
    if (!workspace || !aligned(workspace, 16) || ws_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold fa_bwd_workspace_bytes() = " +
                                          std::to_string(need) + " bytes");
    for (int i = 0; i < 6; ++i)
        if (overlaps(workspace, need, ins[i], in_bytes[i])) return fail(FA_ERR_WORKSPACE, "workspace overlaps an input");
    for (int o = 0; o < 3; ++o)
        if (overlaps(workspace, need, outs[o], out_bytes[o]))
            return fail(FA_ERR_WORKSPACE, "workspace overlaps an output");
    return hip_status(fa::launch_backward(dtype, d, causal != 0, q, k, v, out, dout, lse, dq, dk, dv, B * H, Nq, Nk,
                                          scale, workspace, stream),
                      "backward launch");
}

size_t fa_varlen_workspace_bytes(int num_seqs, int total_q) {
    if (num_seqs < 1 || num_seqs > fa::kMaxVarlenSeqs || total_q < 1) return 0;
    // the tile list: a count, a pad, then (sequence, Q block) pairs; the bound
    // on tiles holds for every Q block size the library uses (>= 128 rows)
    const long long ints = 2 + 2 * fa::varlen_max_tiles(num_seqs, total_q, 128);
    return ((size_t)ints * 4 + 255) / 256 * 256;
}

int fa_fwd_varlen(const void *q, const void *k, const void *v, void *out, float *lse, const int *cu_seqlens_q,
                  const int *cu_seqlens_k, int num_seqs, int total_q, int total_k, int H, int d, float scale,
                  int causal, int dtype, void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "q, k, v, out, cu_seqlens_q and cu_seqlens_k must be non-null");
    if (num_seqs < 1 || total_q < 1 || total_k < 1 || H < 1 || d < 1)
        return fail(FA_ERR_INVALID_ARG, "num_seqs, total_q, total_k, H and d must be >= 1");
    if (!scale_ok(scale)) return fail(FA_ERR_INVALID_ARG, kScaleMsg);
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the variable-length path takes fp16 or bf16");
    if (d != 32 && d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 32, 64 or 128");
    if (num_seqs > fa::kMaxVarlenSeqs) return fail(FA_ERR_UNSUPPORTED, "num_seqs must be <= 4096");
    if ((int64_t)total_q * H * d > INT32_MAX || (int64_t)total_k * H * d > INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "total_q*H*d and total_k*H*d must each fit in 31 bits");
    if ((int64_t)H * fa::varlen_max_tiles(num_seqs, total_q, 128) > INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "too many tiles for one launch");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(FA_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
    if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || (lse && !aligned(lse, 4)))
        return fail(FA_ERR_UNSUPPORTED, "cu_seqlens_q, cu_seqlens_k and lse must be 4-byte aligned");
    const size_t es = element_size(dtype);
    const size_t q_bytes = (size_t)total_q * H * d * es, kv_bytes = (size_t)total_k * H * d * es;
    const size_t lse_bytes = (size_t)H * total_q * 4, cu_bytes = (size_t)(num_seqs + 1) * 4;
    const void *ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
    const size_t in_bytes[5] = {q_bytes, kv_bytes, kv_bytes, cu_bytes, cu_bytes};
    for (int i = 0; i < 5; ++i) {
        if (overlaps(out, q_bytes, ins[i], in_bytes[i])) return fail(FA_ERR_INVALID_ARG, "out overlaps an input");
        if (lse && overlaps(lse, lse_bytes, ins[i], in_bytes[i]))
            return fail(FA_ERR_INVALID_ARG, "lse overlaps an input");
    }
    if (lse && overlaps(lse, lse_bytes, out, q_bytes)) return fail(FA_ERR_INVALID_ARG, "lse overlaps out");
    const size_t need = fa_varlen_workspace_bytes(num_seqs, total_q);
    if (!workspace || !aligned(workspace, 16) || ws_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace must be 16-byte aligned and hold fa_varlen_workspace_bytes() = " +
                                          std::to_string(need) + " bytes");
    for (int i = 0; i < 5; ++i)
        if (overlaps(workspace, need, ins[i], in_bytes[i])) return fail(FA_ERR_WORKSPACE, "workspace overlaps an input");
    if (overlaps(workspace, need, out, q_bytes) || (lse && overlaps(workspace, need, lse, lse_bytes)))
        return fail(FA_ERR_WORKSPACE, "workspace overlaps an output");
    const float sl = (float)((double)scale * kLog2e);
    return hip_status(fa::launch_prefill_varlen(dtype, d, causal != 0, prefill_shape(d), q, k, v, out, lse,
                                                cu_seqlens_q, cu_seqlens_k, num_seqs, H, total_q, total_k, sl,
                                                workspace, stream),
                      "variable-length launch");
}

size_t fa_fp8_pack_bytes(int B, int H, int Nq, int Nk, int d) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
    if ((int64_t)B * H > INT32_MAX) return 0;
    return fa::fp8_layout(B * H, Nq, Nk, d).bytes;
}

// Checks shared by the two FP8 entry points.
static int check_fp8_sizes(int B, int H, int Nq, int Nk, int d) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1)
        return fail(FA_ERR_INVALID_ARG, "B, H, Nq, Nk and d must all be >= 1");
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "the FP8 path takes d = 64 or 128");
    const int64_t nkp = ((int64_t)Nk + 63) / 64 * 64;
    if ((int64_t)B * H > INT32_MAX || (int64_t)Nq * d > INT32_MAX || nkp * d > INT32_MAX)
        return fail(FA_ERR_UNSUPPORTED, "B*H, Nq*d and Nk*d must each fit in 31 bits");
    return FA_OK;
}

int fa_quantize_fp8(const void *q, const void *k, const void *v, const float *signs, int B, int H, int Nq, int Nk,
                    int d, int dtype, void *pack, size_t pack_bytes, hipStream_t stream) {
    if (!q || !k || !v || !pack) return fail(FA_ERR_INVALID_ARG, "q, k, v and pack must be non-null");
    int st = check_fp8_sizes(B, H, Nq, Nk, d);
    if (st != FA_OK) return st;
    if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "the FP8 quantisation takes fp16 or bf16");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(pack, 256))
        return fail(FA_ERR_UNSUPPORTED, "q, k and v must be 16-byte aligned and pack 256-byte aligned");
    if (signs && !aligned(signs, 4)) return fail(FA_ERR_UNSUPPORTED, "signs must be 4-byte aligned");
    const size_t need = fa_fp8_pack_bytes(B, H, Nq, Nk, d);
    if (pack_bytes < need)
        return fail(FA_ERR_WORKSPACE, "pack must hold fa_fp8_pack_bytes() = " + std::to_string(need) + " bytes");
    const size_t bh = (size_t)B * H;
    const size_t q_bytes = bh * Nq * d * 2, kv_bytes = bh * Nk * d * 2;
    if (overlaps(pack, need, q, q_bytes) || overlaps(pack, need, k, kv_bytes) || overlaps(pack, need, v, kv_bytes) ||
        (signs && overlaps(pack, need, signs, (size_t)d * 4)))
        return fail(FA_ERR_INVALID_ARG, "pack overlaps an input");
    return hip_status(fa::launch_fp8_quantize(dtype, d, q, k, v, signs, pack, B * H, Nq, Nk, stream),
                      "FP8 quantisation launch");
}

int fa_fwd_fp8(const void *pack, void *out, float *lse, int B, int H, int Nq, int Nk, int d, float scale,
               int causal, int out_dtype, hipStream_t stream) {
    if (!pack || !out) return fail(FA_ERR_INVALID_ARG, "pack and out must be non-null");
    int st = check_fp8_sizes(B, H, Nq, Nk, d);
    if (st != FA_OK) return st;
    if (!scale_ok(scale)) return fail(FA_ERR_INVALID_ARG, kScaleMsg);
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (out_dtype != FA_F16 && out_dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "out must be fp16 or bf16");
    if (!aligned(pack, 256) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
        return fail(FA_ERR_UNSUPPORTED, "pack must be 256-byte aligned, out 16-byte and lse 4-byte aligned");
    const size_t need = fa_fp8_pack_bytes(B, H, Nq, Nk, d);
    const size_t bh = (size_t)B * H;
    const size_t o_bytes = bh * Nq * d * 2, lse_bytes = bh * Nq * 4;
    if (overlaps(out, o_bytes, pack, need) || (lse && overlaps(lse, lse_bytes, pack, need)) ||
        (lse && overlaps(lse, lse_bytes, out, o_bytes)))
        return fail(FA_ERR_INVALID_ARG, "out and lse must not overlap the pack or each other");
    const float sl = (float)((double)scale * kLog2e);
    return hip_status(fa::launch_fp8_fwd(out_dtype, d, causal != 0, pack, out, lse, B * H, Nq, Nk, sl, stream),
                      "FP8 forward launch");
}

int fa_default_num_splits(int Nk) {
    if (Nk < 1) return 0;
    int s = (Nk + 255) / 256;
    return s < 1 ? 1 : (s > 64 ? 64 : s);
}

int fa_release_workspace(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int status = FA_OK;
    int prev = -1;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    for (auto &kv : g_ws) {
        if (!kv.second.ptr) continue;
        hipError_t err = hipSetDevice(kv.first.first);
        if (err == hipSuccess) err = hipDeviceSynchronize();
        if (err == hipSuccess) err = hipFree(kv.second.ptr);
        if (err != hipSuccess) status = hip_status(err, "releasing a workspace");
        kv.second.ptr = nullptr;
        kv.second.bytes = 0;
    }
    g_ws.clear();
    for (auto &r : g_retired) {
        hipError_t err = hipSetDevice(r.first);
        if (err == hipSuccess) err = hipDeviceSynchronize();
        if (err == hipSuccess) err = hipFree(r.second);
        if (err != hipSuccess) status = hip_status(err, "releasing a workspace");
    }
    g_retired.clear();
    if (have_prev) (void)hipSetDevice(prev);
    return status == FA_OK ? ok() : status;
}

int fa_map_workgroup(int wg, int BH, int Tr, int causal, int *bh, int *qblock) {
    if (BH < 1 || Tr < 1 || (int64_t)BH * Tr > INT32_MAX || wg < 0 || wg >= BH * Tr || !bh || !qblock)
        return fail(FA_ERR_INVALID_ARG, "wg must be in [0, BH*Tr) with BH, Tr >= 1 and non-null outputs");
    fa::layout::map_workgroup(wg, BH, Tr, causal != 0, *bh, *qblock);
    return ok();
}

const char *fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported shape, type or alignment";
        case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        default: return "unknown fa_status";
    }
}

const char *fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return 1; }

}  // extern "C"
