// libtgemm: the attention-forward entry point (C ABI), its argument checks and launch.
// Declarations and conventions are in include/tgemm.h.
#include "tgemm.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attention.hpp"

namespace {

constexpr int64_t kMaxSliceBytes = int64_t(1) << 31;

bool overlap(const void* p, int64_t pb, const void* q, int64_t qb) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return pb > 0 && qb > 0 && a < b + (uintptr_t)qb && b < a + (uintptr_t)pb;
}

}  // namespace

extern "C" int attn_fwd_f16(int64_t batch, int64_t seq, int64_t heads, int64_t dim,
                            const void* Q, const void* K, const void* V, void* O, int causal,
                            void* stream) {
    if (batch < 0 || seq < 0 || heads < 0 || dim < 0 || (causal != 0 && causal != 1))
        return TGEMM_ERR_INVALID_VALUE;
    if (batch == 0 || seq == 0 || heads == 0)
        return TGEMM_OK;
    if (dim != 64)
        return TGEMM_ERR_UNSUPPORTED;
    if (batch > 65535 || heads > 65535 || seq > (int64_t(1) << 30))
        return TGEMM_ERR_UNSUPPORTED;
    // every buffer offset stays below 2^31 bytes
    const int64_t elems = batch * seq * heads * dim;
    if (elems / batch / heads / dim != seq || elems * 2 > kMaxSliceBytes)
        return TGEMM_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O)
        return TGEMM_ERR_NULL_POINTER;
    const auto al16 = [](const void* p) { return ((uintptr_t)p % 16) == 0; };
    if (!al16(Q) || !al16(K) || !al16(V) || !al16(O))
        return TGEMM_ERR_ALIGNMENT;
    const int64_t bytes = elems * 2;
    if (overlap(O, bytes, Q, bytes) || overlap(O, bytes, K, bytes) || overlap(O, bytes, V, bytes))
        return TGEMM_ERR_ALIASING;
    const int nqb = (int)((seq + 127) / 128);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)dim));
    // one workgroup per (query block, batch, head); batch * seq * heads <= 2^24 (the
    // size check above), so the count stays below 2^25
    const dim3 grid((unsigned)(nqb * heads * batch));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const tgemm::u16* q = static_cast<const tgemm::u16*>(Q);
    const tgemm::u16* k = static_cast<const tgemm::u16*>(K);
    const tgemm::u16* v = static_cast<const tgemm::u16*>(V);
    tgemm::u16* o = static_cast<tgemm::u16*>(O);
    if (causal)
        hipLaunchKernelGGL((tgemm::attn_fwd<64, true>), grid, dim3(256), 0, s, q, k, v, o,
                           (int)seq, (int)heads, scale_log2, nqb);
    else
        hipLaunchKernelGGL((tgemm::attn_fwd<64, false>), grid, dim3(256), 0, s, q, k, v, o,
                           (int)seq, (int)heads, scale_log2, nqb);
    return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_LAUNCH;
}
