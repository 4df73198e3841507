// Host-side switch between a compressed and a plain collective: the third
// technique of ZipCCL (abstract, technique (3): the collective is chosen from
// the workload and the system; pith.science, Figure 15 caption: the adaptive
// switcher for reduce-scatter).  The pages give no cost model; the one here
// is the plainest that their workflow supports (pith.science, Figure 5: the
// zipped collectives compress before the exchange and decompress after it,
// and the zipped reduce-scatter is an all-to-all followed by decode and sum).
//
// Per rank, with P ranks, S uncompressed bytes of the collective buffer,
// W = S (P - 1) / P bytes on the wire and W_c = C (P - 1) / P compressed:
//   plain       (P - 1) a + W / B
//   compressed  (P - 1) a + W_c / B + codec time, where the codec time is
//     all-gather      (S / P) / R_comp + W / R_dec   (own shard in, the rest out)
//     all-to-all      S / R_comp + W / R_dec         (one call over all chunks)
//     reduce-scatter  S / R_comp + S / R_red         (all-to-all, then decode + sum)
// Both pay the same step latency, so compression wins exactly when the link
// is slower than B* = (W - W_c) / codec time.
#include <cmath>

#include "zc.h"

namespace {

bool positive(double x) { return std::isfinite(x) && x > 0.0; }

}  // namespace

extern "C" int zc_switch_decide(int32_t collective, int32_t ranks, double bytes,
                                double comp_bytes, const zc_switch_params* p,
                                zc_switch_result* out)
{
    if (!p || !out || ranks < 1 || !(bytes >= 0.0) || !std::isfinite(bytes) ||
        !(comp_bytes >= 0.0) || !std::isfinite(comp_bytes) || (bytes > 0.0 && comp_bytes <= 0.0))
        return ZC_EINVAL;
    if (!positive(p->link_GBps) || !(p->step_latency_us >= 0.0) ||
        !std::isfinite(p->step_latency_us) || !positive(p->compress_GBps))
        return ZC_EINVAL;
    const double P = static_cast<double>(ranks);
    const double S = bytes, B = p->link_GBps * 1e9, a = p->step_latency_us * 1e-6;
    const double Rc = p->compress_GBps * 1e9;
    const double W = S * (P - 1.0) / P, Wc = comp_bytes * (P - 1.0) / P;
    double codec;
    switch (collective) {
    case ZC_COLL_ALLGATHER:
        if (!positive(p->decompress_GBps))
            return ZC_EINVAL;
        codec = (S / P) / Rc + W / (p->decompress_GBps * 1e9);
        break;
    case ZC_COLL_ALLTOALL:
        if (!positive(p->decompress_GBps))
            return ZC_EINVAL;
        codec = S / Rc + W / (p->decompress_GBps * 1e9);
        break;
    case ZC_COLL_REDUCE_SCATTER:
        if (!positive(p->reduce_GBps))
            return ZC_EINVAL;
        codec = S / Rc + S / (p->reduce_GBps * 1e9);
        break;
    default:
        return ZC_EINVAL;
    }
    const double steps = (P - 1.0) * a;
    out->plain_us = (steps + W / B) * 1e6;
    out->compressed_us = (steps + Wc / B + codec) * 1e6;
    if (W <= Wc)
        out->breakeven_GBps = 0.0;
    else if (codec <= 0.0)
        out->breakeven_GBps = INFINITY;
    else
        out->breakeven_GBps = (W - Wc) / codec * 1e-9;
    out->use_compressed = out->compressed_us < out->plain_us ? 1 : 0;
    return ZC_OK;
}
