// Host model of the early-release ring protocol of gemm_early, compiled by
// tests/test_ring_protocol.py with g++ and driven through ctypes.  It replays
// the kernel's own step tables (ring_plan.hpp: kEarlyPrologue, kEarlyLoop,
// load_step, vm_wait, read_ktile) for the four or eight waves of a workgroup over a
// persistent run of `tiles` tiles of `nk` K tiles, and checks the ring's
// hand-offs ("B200 TMA Pipeline Designer", section E step 8: every stage's
// ready and free have a unique producer and consumer; section B: a consumer
// reading right after the load is issued, or a producer overwriting a
// buffer before its readers are done, are the failure modes):
//   ready  every read of a stage (K tile t) or scale-group buffer happens
//          after every wave's direct loads of that content completed (a
//          s_waitcnt vmcnt in the issuing wave) and a barrier followed;
//          every load of K tile t was issued, each exactly once;
//   free   every direct load into a stage or group buffer is issued after
//          every wave's reads of its previous content returned (s_waitcnt
//          lgkmcnt(0) in the reading wave) and a barrier followed;
//   drain  no direct load is in flight when the waves end.
// Direct loads and the epilogue's stores complete in issue order per wave
// (one vmcnt queue); an LDS read completes at the reading wave's next
// lgkmcnt(0) wait.  Every wave runs the same program and every barrier is a
// workgroup barrier, so an event is ordered before another wave's event
// exactly when a barrier separates them (its barrier epoch is lower).
#include <cstdio>
#include <cstring>
#include <deque>
#include <map>
#include <string>
#include <vector>

#include "ring_plan.hpp"

namespace {

using namespace mce;

enum Area { STAGE0 = 0, STAGE1 = 1, GROUP0 = 2, GROUP1 = 3 };

struct Load {
    int area, content, index;   // content: K tile (stages) or group number
    int epoch_issue;
    int epoch_done = -1;        // epoch of the wait that completed it
};

struct Read {
    int area, content;
    int epoch_read;
    int epoch_done = -1;        // epoch of the lgkmcnt(0) wait after it
};

struct Wave {
    std::deque<int> vmq;        // outstanding vm ops: load ids, or -1 for a store
    std::vector<int> pending_reads;
};

struct Model {
    int loads_per_tile, gk, sg;
    std::vector<Load> loads;
    std::vector<Read> reads;
    std::string first_error;
    int errors = 0;

    void error(const std::string &m)
    {
        if (errors++ == 0)
            first_error = m;
    }
};

template <class Op>
int run(const int *pro, int npro, const int *loop, int nloop, int tiles, int nk, int wait_delta,
        char *msg, int msg_len)
{
    using P = EarlyPlan<Op, 256, 256>;
    constexpr int kWaves = P::WAVES;
    constexpr int kGroupLoads = P::GROUP_LOADS;
    Model m;
    m.loads_per_tile = P::LOADS;
    m.gk = P::GK;
    m.sg = Op::SG ? 1 : 0;
    const int total = tiles * nk;   // K tiles the workgroup consumes
    Wave waves[8];
    int epoch = 0;

    auto stage_area = [](int ktile) { return (ktile & 1) ? STAGE1 : STAGE0; };

    auto issue_loads = [&](int w, int area, int content, int lo, int hi) {
        for (int u = lo; u < hi; ++u) {
            Load l{area, content, u, epoch};
            m.loads.push_back(l);
            waves[w].vmq.push_back((int)m.loads.size() - 1);
        }
    };
    auto wait_vm = [&](int w, int keep) {
        auto &q = waves[w].vmq;
        while ((int)q.size() > keep) {
            const int id = q.front();
            q.pop_front();
            if (id >= 0)
                m.loads[id].epoch_done = epoch;
        }
    };
    auto read = [&](int w, int area, int content) {
        m.reads.push_back(Read{area, content, epoch});
        waves[w].pending_reads.push_back((int)m.reads.size() - 1);
    };
    auto wait_lgkm = [&](int w) {
        for (int id : waves[w].pending_reads)
            m.reads[id].epoch_done = epoch;
        waves[w].pending_reads.clear();
    };

    // one step for every wave (they run the same program between barriers)
    auto step = [&](int st, int g) {
        if (st == RS_BARRIER) {
            ++epoch;
            return;
        }
        for (int w = 0; w < kWaves; ++w) {
            LoadStep ls = load_step<P>(st);
            if (ls.ktile > 0) {
                const int t = g + ls.ktile;
                issue_loads(w, stage_area(t), t, ls.lo, ls.hi);
                continue;
            }
            const int vw = vm_wait<P>(st);
            if (vw >= 0) {
                wait_vm(w, vw + wait_delta < 0 ? 0 : vw + wait_delta);
                continue;
            }
            if (st == RS_WAIT_LGKM) {
                wait_lgkm(w);
                continue;
            }
            const int rk = read_ktile(st);
            if (rk >= 0) {
                // (the last phase Y reads K tile `total` too: the stage that
                // the zero-record loads past the last tile filled)
                const int t = g + rk;
                if (st == RS_READ_SCALES && Op::SG)
                    read(w, GROUP0 + group_buffer(t / P::GK), t / P::GK);
                else if (st != RS_READ_SCALES || Op::MX)
                    read(w, stage_area(t), t);
                continue;
            }
            // scale groups: each wave's share, kGroupLoads loads (with
            // eight waves, waves 0-3 load the A rows, 4-7 the B rows: the
            // share is numbered by wave so every load of a group is distinct)
            const int g_lo = kWaves == 8 ? (w >> 2) : 0;
            if (Op::SG && st == RS_ISSUE_GROUP0)
                issue_loads(w, GROUP0 + group_buffer(0), 0, g_lo, g_lo + kGroupLoads);
            if (Op::SG && st == RS_ISSUE_GROUP && g % P::UNR == 0) {
                const int q = g / P::GK + 1;
                issue_loads(w, GROUP0 + group_buffer(q), q, g_lo, g_lo + kGroupLoads);
            }
        }
    };

    for (int i = 0; i < npro; ++i)
        step(pro[i], -1);
    for (int g = 0; g < total; ++g) {
        for (int i = 0; i < nloop; ++i)
            step(loop[i], g);
        if ((g + 1) % nk == 0)
            for (int w = 0; w < kWaves; ++w)   // the tile's epilogue: stores in vmcnt
                for (int s = 0; s < 8; ++s)
                    waves[w].vmq.push_back(-1);
    }
    for (int w = 0; w < kWaves; ++w) {         // the kernel's final vmcnt(0)
        wait_vm(w, 0);
        wait_lgkm(w);
    }

    char buf[256];
    // ready: every read after all loads of its content completed + a barrier
    std::map<std::pair<int, int>, std::vector<int>> by_content;   // (area, content) -> load ids
    for (int id = 0; id < (int)m.loads.size(); ++id)
        by_content[{m.loads[id].area, m.loads[id].content}].push_back(id);
    for (const Read &r : m.reads) {
        auto it = by_content.find({r.area, r.content});
        const int expect = r.area <= STAGE1 ? kWaves * m.loads_per_tile : kWaves * kGroupLoads;
        if (it == by_content.end() || (int)it->second.size() != expect) {
            std::snprintf(buf, sizeof buf, "read of area %d content %d: %d loads issued, %d expected",
                          r.area, r.content, it == by_content.end() ? 0 : (int)it->second.size(),
                          expect);
            m.error(buf);
            continue;
        }
        for (int id : it->second) {
            const Load &l = m.loads[id];
            if (l.epoch_done < 0 || l.epoch_done >= r.epoch_read) {
                std::snprintf(buf, sizeof buf,
                              "ready: read of area %d content %d in epoch %d before load %d "
                              "(issued epoch %d, completed epoch %d) is covered by a wait and a barrier",
                              r.area, r.content, r.epoch_read, l.index, l.epoch_issue, l.epoch_done);
                m.error(buf);
                break;
            }
        }
    }
    // each load index of a content issued exactly once by every wave (stage
    // loads) or once per wave half (eight waves' group loads)
    // (four waves: each issues both indices, A and B rows; eight: waves 0-3
    // index 0, waves 4-7 index 1, so four issues per index either way)
    const int per_index = kWaves * kGroupLoads / 2;
    for (auto &kv : by_content) {
        const bool stage = kv.first.first <= STAGE1;
        std::vector<int> seen(stage ? m.loads_per_tile : 2, 0);
        for (int id : kv.second)
            if (m.loads[id].index < (int)seen.size())
                ++seen[m.loads[id].index];
        // contents that are read must be whole (checked above); none may be
        // loaded twice
        for (int c : seen)
            if (c != 0 && c != (stage ? kWaves : per_index)) {
                std::snprintf(buf, sizeof buf, "area %d content %d: a load issued %d times", kv.first.first,
                              kv.first.second, c / kWaves);
                m.error(buf);
                break;
            }
    }
    // free: every load after every read of the area's previous content
    // returned and a barrier followed
    for (const Load &l : m.loads) {
        const int prev = l.content - 2;
        for (const Read &r : m.reads) {
            if (r.area != l.area || r.content > prev)
                continue;
            if (r.epoch_done < 0 || r.epoch_done >= l.epoch_issue) {
                std::snprintf(buf, sizeof buf,
                              "free: load %d of area %d content %d issued in epoch %d while content %d "
                              "read in epoch %d returns in epoch %d",
                              l.index, l.area, l.content, l.epoch_issue, r.content, r.epoch_read,
                              r.epoch_done);
                m.error(buf);
                break;
            }
        }
    }
    // drain
    for (const Load &l : m.loads)
        if (l.epoch_done < 0) {
            m.error("drain: a direct load still in flight at the end");
            break;
        }
    if (msg && msg_len > 0) {
        std::strncpy(msg, m.first_error.c_str(), msg_len - 1);
        msg[msg_len - 1] = 0;
    }
    return m.errors;
}

} // namespace

extern "C" {

int ring_prologue_steps(int *out)
{
    for (int i = 0; i < kEarlyPrologueSteps; ++i)
        out[i] = kEarlyPrologue[i];
    return kEarlyPrologueSteps;
}

int ring_loop_steps(int *out)
{
    for (int i = 0; i < kEarlyLoopSteps; ++i)
        out[i] = kEarlyLoop[i];
    return kEarlyLoopSteps;
}

int ring_step_id(const char *name)
{
    static const char *names[] = {"READ_TAIL", "ISSUE_PENDING", "MFMA_A", "WAIT_LGKM", "BARRIER",
                                  "ISSUE_X", "MFMA_X", "WAIT_VM", "READ_HEAD", "READ_SCALES",
                                  "ISSUE_Y", "MFMA_Y", "ISSUE_GROUP", "ISSUE_GROUP0", "ISSUE_FIRST",
                                  "ISSUE_SECOND", "WAIT_VM_PRO"};
    static_assert(sizeof(names) / sizeof(names[0]) == RS_NSTEPS, "step names");
    for (int i = 0; i < RS_NSTEPS; ++i)
        if (std::strcmp(names[i], name) == 0)
            return i;
    return -1;
}

// Direct loads of a K tile left for the next phase A (LA)
int ring_pending_loads(int op)
{
    switch (op) {
    case 0: return EarlyPlan<Bf16Ring64, 256, 256>::LA;
    case 1: return EarlyPlan<Bf16Ring64S16, 256, 256>::LA;
    case 7: return EarlyPlan<Bf16Ring64W8, 256, 256>::LA;
    case 8: return EarlyPlan<Bf16Ring64S16W8, 256, 256>::LA;
    case 9: case 10: return EarlyPlan<Mxfp8Ring128GW8, 256, 256>::LA;
    case 2: case 4: return EarlyPlan<Mxfp8Ring128, 256, 256>::LA;
    case 3: case 5: return EarlyPlan<Mxfp8Ring128G, 256, 256>::LA;
    case 6: return EarlyPlan<Fp4Ring128G, 256, 256>::LA;
    default: return -1;
    }
}

// K tiles per scale group (the tiles of a persistent run hold whole groups)
int ring_unroll(int op)
{
    switch (op) {
    case 3: case 5: case 9: case 10: return EarlyPlan<Mxfp8Ring128G, 256, 256>::UNR;
    case 6: return EarlyPlan<Fp4Ring128G, 256, 256>::UNR;
    default: return 1;
    }
}

int ring_model(int op, const int *pro, int npro, const int *loop, int nloop, int tiles, int nk,
               int wait_delta, char *msg, int msg_len)
{
    switch (op) {
    case 0: return run<Bf16Ring64>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 1: return run<Bf16Ring64S16>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 2: return run<Mxfp8Ring128>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 3: return run<Mxfp8Ring128G>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 4: return run<E5m2Ring128>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 5: return run<E5m2Ring128G>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 6: return run<Fp4Ring128G>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 7: return run<Bf16Ring64W8>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 8: return run<Bf16Ring64S16W8>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 9: return run<Mxfp8Ring128GW8>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    case 10: return run<E5m2Ring128GW8>(pro, npro, loop, nloop, tiles, nk, wait_delta, msg, msg_len);
    default: return -1;
    }
}

} // extern "C"
