// decode.hip -- decode attention launch: instantiation choice, split planning
// (one round of workgroups at the kernel's occupancy) and workspace layout
// (counters, then split maxima/sums, then split accumulators).
#include <stdlib.h>

#include <mutex>

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

struct Choice {
    const void* fn;
    int cpl, tile, lds;
};

Choice choose(const Layout& L) {
    Choice c;
    c.tile = (L.G % 64 == 0 && L.gqa == 1) ? 64 : 32;
    // tuning override: KVQ_DECODE_TILE=32|64 (ignored when the key group is not a multiple)
    static const int tile_env = getenv("KVQ_DECODE_TILE") ? atoi(getenv("KVQ_DECODE_TILE")) : 0;
    if ((tile_env == 32 || tile_env == 64) && L.G % tile_env == 0) c.tile = tile_env;
    if (L.D == 128 && L.gqa == 1)
        c.cpl = (L.nvg <= 4) ? 32 : 16;
    else if (L.gqa == 8 && L.bits == 4)
        c.cpl = 8;
    else
        c.cpl = 16;
    switch (L.dtype) {
        case DT_F32: c.fn = dec::decode_kernel_ptr<DT_F32>(L.bits, L.D, L.gqa, c.cpl, c.tile); break;
        case DT_BF16: c.fn = dec::decode_kernel_ptr<DT_BF16>(L.bits, L.D, L.gqa, c.cpl, c.tile); break;
        default: c.fn = dec::decode_kernel_ptr<DT_F16>(L.bits, L.D, L.gqa, c.cpl, c.tile); break;
    }
    // dynamic LDS of the chosen instantiation (see LdsPlan)
    const int wave = (L.gqa * dec::kLimbs * L.D + L.gqa * L.nvg * dec::kLimbs * c.tile + 4 * L.gqa * L.nvg + 15) & ~15;
    const int wg = kWaves * L.gqa * L.D + kWaves * L.gqa * 2 + kMaxCombine + 16 + 4;
    c.lds = kWaves * wave + 4 * wg;
    return c;
}

// workgroups of one instantiation that fit on a CU at once (cached)
int blocks_per_cu(const void* fn, int lds) {
    static std::mutex mu;
    static const void* fns[64];
    static int ldss[64], vals[64], n = 0;
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < n; ++i)
        if (fns[i] == fn && ldss[i] == lds) return vals[i];
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, fn, kThreads, lds) != hipSuccess || v < 1) v = 1;
    if (n < 64) {
        fns[n] = fn;
        ldss[n] = lds;
        vals[n] = v;
        ++n;
    }
    return v;
}
}  // namespace

size_t decode_workspace_bytes(const Layout& L, int max_splits) { return ws_layout(L, max_splits).total; }

bool decode_supported(const Layout& L) { return choose(L).fn != nullptr; }

hipError_t launch_decode(const Layout& L, const DevPtrs& P, const DecodeRequest& rq, const void* q,
                         float* out, float* lse, void* ws, float sm_scale, hipStream_t stream) {
    const Choice ch = choose(L);
    if (!ch.fn) return hipErrorInvalidValue;
    const WsLayout w = ws_layout(L, rq.nsplit_cap);

    // split plan: about one round of workgroups over the whole device, whole key
    // groups per split, a multiple of the wave count when splits are long
    const int64_t ng = rq.Lq / L.G;
    const int cap_q = rq.nsplit_cap;
    int64_t gps = 1;
    if (rq.split_tokens > 0) {
        gps = (rq.split_tokens + L.G - 1) / L.G;
    } else if (ng > 0) {
        const int64_t slots = (int64_t)blocks_per_cu(ch.fn, ch.lds) * rq.num_cu;
        gps = (L.BH * ng + slots - 1) / slots;
        if (gps > kWaves) gps = (gps + kWaves - 1) / kWaves * kWaves;
    }
    if (gps < 1) gps = 1;
    if (ng > 0 && (ng + gps - 1) / gps > cap_q) gps = (ng + cap_q - 1) / cap_q;
    const int nsplit_q = ng > 0 ? (int)((ng + gps - 1) / gps) : 0;
    const int nsplit = nsplit_q > 0 ? nsplit_q : 1;

    dec::DecArgs a;
    a.rec = P.rec;
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
    a.ng_cap = L.ng_cap;
    a.rec_bytes = L.rec_bytes;
    a.rec_kcodes = L.rec_kcodes;
    a.rec_vcodes = L.rec_vcodes;
    a.rec_vmeta = L.rec_vmeta;
    a.Hkv = L.Hkv;
    a.S = L.S;
    a.R = L.R;
    a.nS = (int)rq.nS;
    a.nfp = (int)(rq.nS + rq.r);
    a.G = L.G;
    a.GV = L.GV;
    a.nvg = L.nvg;
    int lg = 0;
    while ((1 << lg) < L.nvg) ++lg;
    a.log2nvg = lg;
    a.gps = (int)gps;
    a.ngroups = (int)ng;
    a.nsplit = nsplit;
    a.nsplit_cap = rq.nsplit_cap;
    a.qscale = sm_scale * 1.4426950408889634f;
    void* args[] = {&a};
    return hipLaunchKernel(ch.fn, dim3((unsigned)nsplit, (unsigned)L.BH), dim3(kThreads), args,
                           (size_t)ch.lds, stream);
}

}  // namespace kvq
