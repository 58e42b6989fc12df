// decode.hip -- decode attention launch: argument packing, tile choice and
// workspace layout (counters, then split maxima/sums, then split accumulators).
#include "decode_dispatch.h"

namespace kvq {

namespace {
struct WsLayout {
    size_t off_counters, off_ml, off_acc, total;
};

WsLayout ws_layout(const Layout& L, int cap) {
    WsLayout w;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    w.off_counters = 0;
    w.off_ml = al((size_t)L.BH * sizeof(unsigned));
    w.off_acc = al(w.off_ml + (size_t)L.BH * cap * L.gqa * 2 * sizeof(float));
    w.total = al(w.off_acc + (size_t)L.BH * cap * L.gqa * L.D * sizeof(float));
    return w;
}
}  // namespace

size_t decode_workspace_bytes(const Layout& L, int max_splits) { return ws_layout(L, max_splits).total; }

hipError_t launch_decode(const Layout& L, const DevPtrs& P, const DecodePlan& plan, const void* q,
                         float* out, float* lse, void* ws, float sm_scale, hipStream_t stream,
                         int nsplit_cap) {
    const WsLayout w = ws_layout(L, nsplit_cap);
    dec::DecArgs a;
    a.kcodes = P.kcodes;
    a.vcodes = P.vcodes;
    a.kmeta = P.kmeta;
    a.vmeta = P.vmeta;
    a.ksink = P.ksink;
    a.vsink = P.vsink;
    a.kres = P.kres;
    a.vres = P.vres;
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.counters = reinterpret_cast<unsigned*>((char*)ws + w.off_counters);
    a.part_ml = reinterpret_cast<float*>((char*)ws + w.off_ml);
    a.part_acc = reinterpret_cast<float*>((char*)ws + w.off_acc);
    a.Lq_cap = L.Lq_cap;
    a.ng_cap = L.ng_cap;
    a.Lq = plan.Lq;
    a.Hkv = L.Hkv;
    a.S = L.S;
    a.R = L.R;
    a.nS = plan.nS;
    a.r = plan.r;
    a.G = L.G;
    a.GV = L.GV;
    a.nvg = L.nvg;
    a.gps = plan.gps;
    a.nsplit_q = plan.nsplit_q;
    a.nsplit = plan.nsplit;
    a.nsplit_cap = nsplit_cap;
    a.has_fp = plan.has_fp;
    a.qscale = sm_scale * 1.4426950408889634f;
    const int tile = (L.G % 64 == 0) ? 64 : 32;
    int cpl = 16;
    if (L.D == 128 && L.gqa == 1 && L.GV % 32 == 0) cpl = 32;
    if (L.gqa == 8 && L.bits == 4) cpl = 8;
    dim3 grid((unsigned)plan.nsplit, (unsigned)L.BH);
    switch (L.dtype) {
        case DT_F32: return dec::launch_decode_dt<DT_F32>(a, L.bits, L.D, L.gqa, cpl, tile, grid, stream);
        case DT_BF16: return dec::launch_decode_dt<DT_BF16>(a, L.bits, L.D, L.gqa, cpl, tile, grid, stream);
        default: return dec::launch_decode_dt<DT_F16>(a, L.bits, L.D, L.gqa, cpl, tile, grid, stream);
    }
}

}  // namespace kvq
