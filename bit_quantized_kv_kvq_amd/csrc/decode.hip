// decode.hip -- decode attention launch: instantiation choice, split planning
// (about one workgroup per CU), the split combine's grouping and the workspace
// layout (counters, then split maxima/sums and accumulators, then those of the
// combine's groups).
#include <hip/hip_ext.h>

#include <mutex>

#include "decode_dispatch.h"

namespace kvq {

namespace {
// Splits per slice up to which the slice's last arrival merges them all; above
// it, groups of about sqrt(nsplit) splits merge first (two-level combine).  Both
// keep every merge within kMaxMerge partials for nsplit <= kMaxSplits.
constexpr int kOneLevelSplits = kMaxMerge;
static_assert(kOneLevelSplits <= kMaxMerge, "one-level combine within a merge");

int ceil_sqrt(int n) {
    int s = 0;
    while (s * s < n) ++s;
    return s;
}
// splits per first-level group for nsplit splits (>= nsplit: one level)
int combine_group(int nsplit) { return nsplit > kOneLevelSplits ? ceil_sqrt(nsplit) : nsplit; }
// groups of any split count up to cap: ceil(n / ceil(sqrt n)) <= ceil(sqrt n)
int combine_groups_cap(int cap) { return cap > kOneLevelSplits ? ceil_sqrt(cap) : 1; }

struct WsLayout {
    size_t off_counters, off_ml, off_acc, off_gml, off_gacc, total;
    int gcap;
};

WsLayout ws_layout(const Layout& L, int cap) {
    WsLayout w;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    w.gcap = combine_groups_cap(cap);
    w.off_counters = 0;
    w.off_ml = al((size_t)L.BH * (1 + w.gcap) * sizeof(unsigned));
    w.off_acc = al(w.off_ml + (size_t)L.BH * cap * L.gqa * 2 * sizeof(float));
    w.off_gml = al(w.off_acc + (size_t)L.BH * cap * L.gqa * L.D * sizeof(float));
    w.off_gacc = al(w.off_gml + (size_t)L.BH * w.gcap * L.gqa * 2 * sizeof(float));
    w.total = al(w.off_gacc + (size_t)L.BH * w.gcap * L.gqa * L.D * sizeof(float));
    return w;
}

struct Choice {
    const void* fn;
    int cpl, tile, tpg, lds;
    int occ;  // workgroups per CU the kernel is planned for
    bool mf;  // the quantized stream runs on the matrix cores
};

Choice choose(const Layout& L) {
    Choice c;
    c.tile = (L.gqa == 1 && L.G >= 64) ? 64 : 32;
    c.tpg = L.G / c.tile;
    if (L.D == 128 && L.gqa == 1)
        c.cpl = (L.nvg <= 4) ? 32 : 16;
    else if (L.gqa == 8 && L.bits == 4)
        c.cpl = 8;
    else
        c.cpl = 16;
    c.fn = nullptr;
    c.occ = 1;
    c.mf = false;
    if (c.tile * c.tpg == L.G) {
        if (L.bits == 4 && L.D == 128) c.fn = dec::decode_kernel_ptr<4, 128>(L.gqa, c.cpl, c.tile, c.tpg);
        if (L.bits == 2 && L.D == 128) c.fn = dec::decode_kernel_ptr<2, 128>(L.gqa, c.cpl, c.tile, c.tpg);
        if (L.bits == 4 && L.D == 64) c.fn = dec::decode_kernel_ptr<4, 64>(L.gqa, c.cpl, c.tile, c.tpg);
        if (L.bits == 2 && L.D == 64) c.fn = dec::decode_kernel_ptr<2, 64>(L.gqa, c.cpl, c.tile, c.tpg);
    }
    // dynamic LDS of the chosen instantiation (see LdsPlan)
    int wave = (L.gqa * dec::kLimbs * L.D + 2 * L.gqa * L.nvg * dec::kLimbs * c.tile + 15) & ~15;
    // Several query heads per kv head (or 8-bit codes), key groups of 64 to 256
    // tokens and value groups of 64 channels or more: the quantized stream runs on
    // the matrix cores.
    if ((L.gqa >= 2 || L.bits == 8) && L.G >= 64 && L.G <= 256 && L.GV >= 64 && (L.D == 128 || L.nvg == 1)) {
        const void* mf = nullptr;
        const int tpg = L.G / 64;
        if (L.bits == 4 && L.D == 128) mf = dec::decode_mf_kernel_ptr<4, 128>(L.gqa, tpg, L.nvg);
        if (L.bits == 2 && L.D == 128) mf = dec::decode_mf_kernel_ptr<2, 128>(L.gqa, tpg, L.nvg);
        if (L.bits == 4 && L.D == 64) mf = dec::decode_mf_kernel_ptr<4, 64>(L.gqa, tpg, L.nvg);
        if (L.bits == 2 && L.D == 64) mf = dec::decode_mf_kernel_ptr<2, 64>(L.gqa, tpg, L.nvg);
        if (L.bits == 8 && L.D == 128) mf = dec::decode_mf_kernel_ptr<8, 128>(L.gqa, tpg, L.nvg);
        if (L.bits == 8 && L.D == 64) mf = dec::decode_mf_kernel_ptr<8, 64>(L.gqa, tpg, L.nvg);
        if (mf != nullptr) {
            c.fn = mf;
            c.mf = true;
            c.occ = dec::two_waves(true, L.bits, L.gqa, false) ? 2 : 1;
            c.tile = 64;
            c.tpg = tpg;
            const int rbk = (L.gqa + 3) / 4;
            wave = rbk * (L.D / 64) * 1024 + 2 * L.nvg * rbk * 1024;  // MStream::lds_bytes
        }
    }
    if (L.outliers) {
        // dense-and-sparse records, with their outlier terms (LdsPlan's SPB): on the
        // matrix cores where the plain cache would be (head_dim 128), else the VALU
        // stream (32-token tiles for several query heads per kv head)
        c.fn = nullptr;
        c.occ = 1;
        c.mf = false;
        const int spb = 4 * (L.gqa * L.G + L.gqa * L.D);
        if (L.gqa >= 2 && L.G >= 64 && L.G <= 256 && L.GV >= 64 && L.D == 128 && L.bits != 8) {
            c.mf = true;
            c.tile = 64;
            c.tpg = L.G / 64;
            c.occ = dec::two_waves(true, L.bits, L.gqa, true) ? 2 : 1;
            if (L.bits == 4) c.fn = dec::decode_mfsp_kernel_ptr<4>(L.gqa, c.tpg, L.nvg);
            if (L.bits == 2) c.fn = dec::decode_mfsp_kernel_ptr<2>(L.gqa, c.tpg, L.nvg);
            const int rbk = (L.gqa + 3) / 4;
            wave = rbk * (L.D / 64) * 1024 + 2 * L.nvg * rbk * 1024 + spb;  // MStream::lds_bytes + SPB
        } else {
            c.tile = (L.gqa == 1 && L.G >= 64) ? 64 : 32;  // the VALU map (the matrix-core choice may have set 64)
            c.tpg = L.G / c.tile;
            if (c.tile * c.tpg == L.G) {
                c.occ = dec::two_waves(false, L.bits, L.gqa, true) ? 2 : 1;
                if (L.bits == 4 && L.D == 128) c.fn = dec::decode_sp_kernel_ptr<4, 128>(L.gqa, c.cpl, c.tile, c.tpg, L.nvg);
                if (L.bits == 2 && L.D == 128) c.fn = dec::decode_sp_kernel_ptr<2, 128>(L.gqa, c.cpl, c.tile, c.tpg, L.nvg);
                if (L.bits == 4 && L.D == 64) c.fn = dec::decode_sp_kernel_ptr<4, 64>(L.gqa, c.cpl, c.tile, c.tpg, L.nvg);
                if (L.bits == 2 && L.D == 64) c.fn = dec::decode_sp_kernel_ptr<2, 64>(L.gqa, c.cpl, c.tile, c.tpg, L.nvg);
            }
            wave = ((L.gqa * dec::kLimbs * L.D + 2 * L.gqa * L.nvg * dec::kLimbs * c.tile + 15) & ~15) + spb;
        }
    }
    if (L.key_axis) {
        // per-token keys (64-token tiles, one or two per record): on the matrix cores
        // where the per-channel cache would be, else the VALU stream for one query head
        // per kv head; other shapes have no kernel
        c.fn = nullptr;
        c.occ = 1;
        c.mf = false;
        c.tile = 64;
        c.tpg = L.G / 64;
        const bool mf = (L.gqa >= 2 || L.bits == 8) && L.GV >= 64 && (L.D == 128 || L.nvg == 1);
        const void* kt = nullptr;
        if (mf || (L.gqa == 1 && L.bits != 8)) {
            if (L.bits == 2 && L.D == 128) kt = dec::decode_kt_kernel_ptr<2, 128>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
            if (L.bits == 4 && L.D == 128) kt = dec::decode_kt_kernel_ptr<4, 128>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
            if (L.bits == 8 && L.D == 128) kt = dec::decode_kt_kernel_ptr<8, 128>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
            if (L.bits == 2 && L.D == 64) kt = dec::decode_kt_kernel_ptr<2, 64>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
            if (L.bits == 4 && L.D == 64) kt = dec::decode_kt_kernel_ptr<4, 64>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
            if (L.bits == 8 && L.D == 64) kt = dec::decode_kt_kernel_ptr<8, 64>(L.gqa, c.cpl, c.tpg, L.nvg, mf);
        }
        if (kt != nullptr) {
            c.fn = kt;
            c.mf = mf;
            c.occ = dec::two_waves(mf, L.bits, L.gqa, false) ? 2 : 1;
            if (mf) {
                const int rbk = (L.gqa + 3) / 4;
                wave = rbk * (L.D / 64) * 1024 + 2 * L.nvg * rbk * 1024;  // MStream::lds_bytes
            } else {
                wave = (L.gqa * dec::kLimbs * L.D + 2 * L.gqa * L.nvg * dec::kLimbs * c.tile + 15) & ~15;
            }
        }
    }
    const int wg = kWaves * L.gqa * L.D + kWaves * L.gqa * 2 + 4;  // LdsPlan::wg_floats
    c.lds = kWaves * wave + 4 * wg;
    return c;
}

}  // namespace

size_t decode_workspace_bytes(const Layout& L, int max_splits) { return ws_layout(L, max_splits).total; }

namespace {
// The decode workspace of callers that cannot allocate.  In host code `scratch`
// names a host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ __launch_bounds__(256) void clear_words_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}
}  // namespace

hipError_t static_scratch(hipStream_t stream, void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        clear_words_kernel<<<1024, 256, 0, stream>>>(static_cast<uint4*>(p), kStaticScratchBytes / 16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool decode_supported(const Layout& L) { return choose(L).fn != nullptr; }

hipError_t launch_decode(const Layout& L, const DevPtrs& P, const DecodeRequest& rq, const void* q,
                         float* out, float* lse, void* ws, float sm_scale, hipStream_t stream) {
    const Choice ch = choose(L);
    if (!ch.fn) return hipErrorInvalidValue;
    const WsLayout w = ws_layout(L, rq.nsplit_cap);

    // Split plan: about one workgroup per CU (two for the streams that run two
    // waves per SIMD), whole key groups per split, a multiple of the wave count
    // when splits are long.  Long per-wave streams beat more workgroups per CU:
    // every stream pays a start-up latency and the split combine, while the
    // prefetch ring already covers the memory latency at one workgroup per CU.
    const int64_t ng = rq.Lq / L.G;
    const int cap_q = rq.nsplit_cap;
    int64_t gps = 1;
    if (rq.split_tokens > 0) {
        gps = (rq.split_tokens + L.G - 1) / L.G;
    } else if (ng > 0) {
        // Sequences of different lengths: planned for the longest (splitting by
        // the total over all slices measured slower: more workgroups and combines).
        const int64_t slots = (int64_t)rq.num_cu * ch.occ;
        gps = (L.BH * ng + slots - 1) / slots;
        if (gps > kWaves) gps = (gps + kWaves - 1) / kWaves * kWaves;
    }
    if (gps < 1) gps = 1;
    if (ng > 0 && (ng + gps - 1) / gps > cap_q) gps = (ng + cap_q - 1) / cap_q;
    // Paged records: a split spans at most 64 pages (one lane each), which
    // gps <= 63 P guarantees; the cache's split capacity admits it.
    if (L.lp >= 0 && gps > 63 * ((int64_t)1 << L.lp)) gps = 63 * ((int64_t)1 << L.lp);
    const int nsplit_q = ng > 0 ? (int)((ng + gps - 1) / gps) : 0;
    const int nsplit = nsplit_q > 0 ? nsplit_q : 1;
    // nsplit <= nsplit_cap <= kMaxSplits: every merge of the combine takes at most
    // kMaxMerge partials
    if (nsplit > kMaxSplits) return hipErrorInvalidValue;

    // Split weights.  With two workgroups per CU and a grid that fills every slot
    // exactly once, the workgroup dispatched first on a CU runs ahead of the one
    // dispatched second: its waves are older and win the SIMDs' issue arbitration
    // (per-workgroup timestamps: 33 against 42.5 us of stream on the LogQuant
    // decode, 20 against 26 us on the long-context one, on every CU).  Workgroups
    // take one slot on every CU, in dispatch order, before any CU takes a second,
    // and the grid is split-major, so splits below num_cu / BH run first on their
    // CUs; they take 11/8 of the others' key groups, so that both end together.
    // This is done for the matrix-core stream (on the VALU stream's outlier kernel,
    // the one other stream run two per CU, it measured 1% slower).  Otherwise (and
    // for paged records, whose splits are bounded in pages, or a fixed split size)
    // every split takes gps groups and the grid is slice-major.  The kernels compile
    // the weighted plan exactly where ch.mf && ch.occ == 2 (their WSPLIT).
    int s1 = nsplit;
    int64_t gps2 = gps;
    if (ch.mf && ch.occ == 2 && L.lp < 0 && rq.split_tokens == 0 && nsplit > 1 && ng > 0 &&
        (int64_t)nsplit * L.BH == 2 * (int64_t)rq.num_cu && rq.num_cu % L.BH == 0) {
        s1 = nsplit / 2;  // = num_cu / BH
        const int64_t pair = (ng + s1 - 1) / s1;  // groups of a first and a second split
        const int64_t g1 = (pair * 11 + 9) / 19;
        if (g1 >= 1 && pair - g1 >= 1) {
            gps = g1;
            gps2 = pair - g1;
        } else {
            s1 = nsplit;
        }
    }

    dec::DecArgs a;
    a.rec = P.rec;
    a.ksink = P.ksink;
    a.vsink = P.vsink;
    a.kres = P.kres;
    a.vres = P.vres;
    a.knew = static_cast<const char*>(rq.knew);
    a.vnew = static_cast<const char*>(rq.vnew);
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.counters = reinterpret_cast<unsigned*>((char*)ws + w.off_counters);
    a.part_ml = reinterpret_cast<float*>((char*)ws + w.off_ml);
    a.part_acc = reinterpret_cast<float*>((char*)ws + w.off_acc);
    a.grp_ml = reinterpret_cast<float*>((char*)ws + w.off_gml);
    a.grp_acc = reinterpret_cast<float*>((char*)ws + w.off_gacc);
    a.cgroups_cap = w.gcap;
    a.ng_cap = L.ng_cap;
    a.rec_bytes = L.rec_bytes;
    a.rec_kcodes = L.rec_kcodes;
    a.rec_vcodes = L.rec_vcodes;
    a.rec_vmeta = L.rec_vmeta;
    a.rec_kov = L.rec_kov;
    a.rec_koi = L.rec_koi;
    a.rec_vov = L.rec_vov;
    a.rec_voi = L.rec_voi;
    a.Hkv = L.Hkv;
    a.S = L.S;
    a.R = L.R;
    a.Qf = L.Qf;
    a.nS = (int)rq.nS;
    a.nfp = (int)(rq.nS + rq.r);
    a.G = L.G;
    a.dtype = L.dtype;
    a.GV = L.GV;
    a.nvg = L.nvg;
    a.gps = (int)gps;
    a.s1 = s1;
    a.gps2 = (int)gps2;
    a.split_major = s1 < nsplit ? 1 : 0;
    a.ngroups = (int)ng;
    a.nsplit = nsplit;
    a.nsplit_cap = rq.nsplit_cap;
    a.cgs = combine_group(nsplit);
    a.qscale = sm_scale * 1.4426950408889634f;
    a.base_len = rq.rg.base_len;
    a.len_delta = rq.rg.delta;
    a.table = P.table;
    a.lp = L.lp;
    a.max_pages = (int)L.max_pages;
    a.pool_pages = (int)L.pool_pages;
    a.page_bytes = (uint32_t)L.page_bytes;
    a.pool_bytes = (uint32_t)(L.pool_pages * L.page_bytes);
    void* args[] = {&a};
    const dim3 grid = a.split_major ? dim3((unsigned)L.BH, (unsigned)nsplit) : dim3((unsigned)nsplit, (unsigned)L.BH);
    if (rq.ev_start != nullptr)
        return hipExtLaunchKernel(ch.fn, grid, dim3(kThreads), args, (size_t)ch.lds, stream, rq.ev_start,
                                  rq.ev_stop, 0);
    return hipLaunchKernel(ch.fn, grid, dim3(kThreads), args, (size_t)ch.lds, stream);
}

}  // namespace kvq
