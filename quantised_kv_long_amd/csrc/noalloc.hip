// noalloc.hip -- kvq_decode_step_noalloc: the decode step with its split
// partials in a file-scope device array instead of caller memory, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in the library's code object: each GPU the library runs on
// holds its own copy from module load until the process ends.  Host code never
// passes the array's name to a kernel (in host code it is only a stand-in for
// the symbol): the first call on a device, with that device current, looks up
// the device address with hipGetSymbolAddress and keeps it per device; every
// later use goes through that address.
#include <mutex>

#include <hip/hip_runtime.h>

#include "kvq.h"
#include "kvq_internal.hpp"

namespace {

// the split partials of one call: part_o at offset 0, part_lse after it (at a
// 256-byte boundary)
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
void* g_scratch[MAX_DEVICES];   // device address of `scratch` per device (null: not looked up yet)

// The device address of this device's array; null when the lookup fails.
void* scratch_ptr(int dev)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

}  // namespace

extern "C" {

size_t kvq_decode_step_noalloc_bytes(int B, int Hq, int D, int max_seq_len, int split_tokens)
{
    if (B < 1 || Hq < 1 || D < 1 || max_seq_len < 1 || split_tokens < 1) return 0;
    const size_t S = ((size_t)max_seq_len + split_tokens - 1) / split_tokens;
    return round_up((size_t)B * Hq * S * D * sizeof(float), 256) + (size_t)B * Hq * S * sizeof(float);
}

int kvq_decode_step_noalloc(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                            const void* v_new, const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv,
                            int D, float softmax_scale, int max_seq_len, int split_tokens, int out_type, void* out,
                            float* lse_out, void* stream)
{
    // every check of kvq_decode_step (with the partials this call would use)
    // and the scratch size, before any HIP call
    if (B < 1 || Hq < 1 || D < 1 || max_seq_len < 1) return KVQ_ERR_SHAPE;
    if (split_tokens < KVQ_SPLIT_GRANULE || split_tokens % KVQ_SPLIT_GRANULE != 0) return KVQ_ERR_SPLITS;
    const int64_t max_splits64 = ((int64_t)max_seq_len + split_tokens - 1) / split_tokens;
    if (max_splits64 > 65535) return KVQ_ERR_SPLITS;
    const int max_splits = (int)max_splits64;
    // stand-ins with the alignment the scratch partials have (nothing is
    // dereferenced by the checks)
    const float* o_chk = reinterpret_cast<const float*>((uintptr_t)256);
    const float* l_chk = reinterpret_cast<const float*>((uintptr_t)256);
    const int rc = kvq::validate_step(k_cache, v_cache, k_new, v_new, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                      max_seq_len, split_tokens, max_splits, o_chk, l_chk, out_type, out, lse_out);
    if (rc != KVQ_OK) return rc;
    const size_t need = kvq_decode_step_noalloc_bytes(B, Hq, D, max_seq_len, split_tokens);
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_CAPACITY;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return KVQ_ERR_LAUNCH;
    unsigned char* base = static_cast<unsigned char*>(scratch_ptr(dev));
    if (!base) return KVQ_ERR_LAUNCH;
    float* part_o = reinterpret_cast<float*>(base);
    float* part_lse =
        reinterpret_cast<float*>(base + round_up((size_t)B * Hq * max_splits * D * sizeof(float), 256));
    return kvq_decode_step(k_cache, v_cache, k_new, v_new, q, seq_lens, B, Hq, Hkv, D, softmax_scale, max_seq_len,
                           split_tokens, max_splits, part_o, part_lse, out_type, out, lse_out, stream);
}

}  // extern "C"
