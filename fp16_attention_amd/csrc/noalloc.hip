// The allocation-free decode entry point, attn_fwd_paged_e4m3_decode_noalloc.
//
// For callers that cannot allocate device memory: code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc. It is the
// paged E4M3 decode of attn_fwd_paged_e4m3_decode, whose split-KV partial
// states (FP32 unnormalised output, running maximum and sum per key segment)
// go to a file-scope device array of the library instead of a caller
// workspace.
//
// The array below is what each GPU the library runs on holds from module load
// until the process ends. In host code its name is only a host-side stand-in:
// the device address comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the entry point's first call there, and kept
// in scratch_ptr; host code passes only that address to kernels.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, or two host threads) race. Nothing in it has to start at
// zero: every partial state the merge reads is written by the same call first
// (a segment past a query tile's keys is neither written nor read).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa16attn.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices];  // per device: the address of `scratch` there

// The current device's address of the scratch array (looked up once per device).
int scratch_ptr(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return FA_ERR_HIP + (int)e;
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_scratch_lock);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return FA_ERR_HIP + (int)e;
        if (!p) return FA_ERR_HIP + (int)hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

// WorkspaceSource for the launcher: the scratch array, if the call's partial
// states fit it (checked before any HIP call).
int scratch_workspace(size_t need, void** ptr, size_t* bytes)
{
    if (need > kScratchBytes) return FA_ERR_WORKSPACE;
    const int rc = scratch_ptr(ptr);
    if (rc) return rc;
    *bytes = kScratchBytes;
    return FA_OK;
}

const fa::WorkspaceSource kScratchSource = {scratch_workspace};

}  // namespace

extern "C" int attn_fwd_paged_e4m3_decode_noalloc(fa_tensor q, const uint8_t* k_cache, const uint8_t* v_cache,
                                                  const int32_t* page_table, int64_t table_stride,
                                                  int num_phys_pages, int page_size, float k_scale, float v_scale,
                                                  fa_tensor o, float* lse, int B, int Hq, int Hkv, int D,
                                                  int q_rows, int q_real, int kv_len, float scale, void* stream)
{
    return fa::paged_decode_from(&kScratchSource, q.data, q.stride_b, q.stride_h, q.stride_s, k_cache, v_cache,
                                 page_table, table_stride, num_phys_pages, page_size, k_scale, v_scale, o.data,
                                 o.stride_b, o.stride_h, o.stride_s, lse, B, Hq, Hkv, D, q_rows, q_real, kv_len,
                                 scale, stream);
}
