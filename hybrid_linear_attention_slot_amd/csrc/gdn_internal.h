// Host-side internals of the GDN state library: the pool handle, error
// reporting and the kernel launchers each .hip file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <vector>

#include "gdn.h"

struct gdn_pool {
    gdn_pool_desc desc;          // desc.layer_base points at `bases`
    std::vector<void*> bases;    // copy of the caller's layer table
    std::vector<int32_t> linear; // indices of layers with a state pool
    int64_t ssm_bytes;           // Hv*dk*dv*4
    int64_t conv_bytes;          // (W-1)*C*2
};

namespace gdn {

// Record `code` with a printf-style message for gdn_last_error(); returns code.
// Allocates nothing (a fixed per-thread buffer), so it is safe under memory
// exhaustion.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int check_launch(const char* what); // GDN_OK, or GDN_EHIP after a launch error

// Runs f(), which returns a GDN code; a host allocation failure becomes
// GDN_ENOMEM and any other C++ exception GDN_EINVAL, so that none crosses the
// C ABI.
template <class F>
int guarded(F&& f) noexcept
{
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return fail(GDN_ENOMEM, "out of host memory");
    } catch (...) {
        return fail(GDN_EINVAL, "internal error");
    }
}

// ---- restore / gather / scatter (copy_kernels.hip) ----------------------
struct HitPair {
    int32_t dst;
    int32_t src;
};
struct HsWrite {
    int32_t row;
    int32_t value;
};
// Copies every pair over every layer in `layers` (indices into the pool's
// layer table) and writes the hs entries; splits into launches that fit the
// kernel-argument budget.
int launch_restore(const gdn_pool* pool, const std::vector<HitPair>& pairs,
                   const std::vector<HsWrite>& hs, uint8_t* hs_dev, hipStream_t stream);
int launch_gather(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                  void* ssm_dense, void* conv_dense, hipStream_t stream);
int launch_scatter(const gdn_pool* pool, int32_t layer, const int32_t* idx, int32_t n,
                   const void* ssm_dense, const void* conv_dense, hipStream_t stream);

// ---- decode / prefill (decode_kernel.hip, prefill_kernel.hip) ----------
bool decode_supported(int dk, int dv, int W);
bool prefill_supported(int dk, int dv, int W);
int launch_decode(const gdn_pool* pool, int32_t layer, int32_t rows, const gdn_step_args* a,
                  hipStream_t stream);
// ckpt_slot / ckpt_len: NULL, or device int32 [num_seqs] (checkpoint emission)
int launch_prefill(const gdn_pool* pool, int32_t layer, int32_t num_seqs, int64_t total_tokens,
                   const int32_t* cu, const gdn_step_args* a, const int32_t* ckpt_slot,
                   const int32_t* ckpt_len, hipStream_t stream);

} // namespace gdn
