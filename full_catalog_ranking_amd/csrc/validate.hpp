// Host-side argument checks of the C ABI (see include/genrec.h for each entry
// point's contract).  Pure C++ (no HIP): the library's entry points call
// these before any launch, and the host test build runs them under the
// address and undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/genrec.h"

namespace genrec {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shape / pointer checks of the ranking-head entry points.  Returns GENREC_OK
// or the status to report; never touches the device.
inline int check_common(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                        const int32_t* out_idx, const float* out_scores, const float* out_lse) {
    if (dtype != GENREC_BF16 && dtype != GENREC_F32) return GENREC_ERR_INVALID_ARG;
    if (B <= 0 || D <= 0 || M <= 0 || K <= 0) return GENREC_ERR_INVALID_ARG;
    if (!H || !E || !out_idx || !out_scores || !out_lse) return GENREC_ERR_INVALID_ARG;
    if (!aligned(H, 16) || !aligned(E, 16)) return GENREC_ERR_INVALID_ARG;
    if (!aligned(out_idx, 4) || !aligned(out_scores, 4) || !aligned(out_lse, 4))
        return GENREC_ERR_INVALID_ARG;
    if (K > GENREC_KMAX) return GENREC_ERR_UNSUPPORTED;
    if (M >= ((int64_t)1 << 31)) return GENREC_ERR_UNSUPPORTED;
    if (D % (dtype == GENREC_BF16 ? 8 : 4) != 0) return GENREC_ERR_UNSUPPORTED;
    if (D > GENREC_DMAX) return GENREC_ERR_UNSUPPORTED;
    return GENREC_OK;
}

// The same for the cross-entropy entry points (bf16 only).
inline int check_ce(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels,
                    const float* weights) {
    if (B <= 0 || D <= 0 || M <= 0) return GENREC_ERR_INVALID_ARG;
    if (!H || !E || !labels) return GENREC_ERR_INVALID_ARG;
    if (!aligned(H, 16) || !aligned(E, 16) || !aligned(labels, 4) || (weights && !aligned(weights, 4)))
        return GENREC_ERR_INVALID_ARG;
    if (M >= ((int64_t)1 << 31)) return GENREC_ERR_UNSUPPORTED;
    if (D % 8 != 0 || D > GENREC_DMAX) return GENREC_ERR_UNSUPPORTED;
    return GENREC_OK;
}

}  // namespace genrec
