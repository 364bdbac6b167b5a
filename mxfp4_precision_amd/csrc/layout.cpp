// Host-side conversion of one blob between MX_LAYOUT_CANONICAL and
// MX_LAYOUT_TILED (layout definitions in include/mxfp4.h).  Works a 16-byte
// lane slice at a time: a slice is 32 consecutive elements (one k-block) of
// one row in both layouts, so the data conversion is a block copy.

#include <cstring>

#include "mx_internal.h"

extern "C" mx_status mx_layout_convert_host(int to_tiled, int64_t rows, int64_t length, const void *q_src,
                                            const void *s_src, void *q_dst, void *s_dst) {
    if (rows < 0 || length < 0) return MX_ERR_INVALID_ARGUMENT;
    if (!q_src || !s_src || !q_dst || !s_dst) return MX_ERR_INVALID_ARGUMENT;
    const int64_t Lp = mx::padded(length);
    const int64_t nblk = Lp / 32;              // k-blocks per row
    const int64_t ksteps = Lp / 128;
    const int64_t kgroups = mx::cdiv(Lp, 512);
    const int64_t r16 = mx::cdiv(rows, 16) * 16;
    const uint8_t *qs = static_cast<const uint8_t *>(q_src);
    const uint8_t *ss = static_cast<const uint8_t *>(s_src);
    uint8_t *qd = static_cast<uint8_t *>(q_dst);
    uint8_t *sd = static_cast<uint8_t *>(s_dst);
    if (to_tiled) {
        std::memset(qd, 0, (size_t)(r16 * Lp / 2));
        std::memset(sd, 0, (size_t)(r16 * kgroups * 16));
    }
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t g = r / 16, rr = r % 16;
        for (int64_t kb = 0; kb < nblk; ++kb) {
            const int64_t canon_q = r * (Lp / 2) + kb * 16;
            const int64_t tiled_q = (g * ksteps + kb / 4) * 1024 + (rr + 16 * (kb % 4)) * 16;
            const int64_t canon_s = r * nblk + kb;
            const int64_t tiled_s = (g * kgroups + kb / 16) * 256 + 4 * (rr + 16 * (kb % 4)) + (kb % 16) / 4;
            if (to_tiled) {
                std::memcpy(qd + tiled_q, qs + canon_q, 16);
                sd[tiled_s] = ss[canon_s];
            } else {
                std::memcpy(qd + canon_q, qs + tiled_q, 16);
                sd[canon_s] = ss[tiled_s];
            }
        }
    }
    return MX_SUCCESS;
}
