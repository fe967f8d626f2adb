// kvq_nodev.cpp -- recording launcher for CPU tests of the host library.
//
// libkvq_nodev.so is kvq_host.cpp linked against this file instead of the
// HIP kernels: every launch is appended as one text line to a log instead of
// running, so tests can check validation, the ring planner and the split-K
// plan without a GPU.  kvq_nodev_fail_next() makes the next launch report a
// failure, to exercise the KVQ_EDEVICE path.
#include <cstdio>
#include <string>

#include "kvq_internal.h"

namespace {
std::string g_log;
int g_fail_next = 0;
int g_cus = 256;   // the compute units a handle sees (MI355X: 256)

int record(const std::string& line, const char** err) {
    if (g_fail_next) {
        g_fail_next = 0;
        *err = "simulated launch failure";
        return 1;
    }
    g_log += line;
    g_log += '\n';
    return 0;
}
}  // namespace

namespace kvq {

int device_compute_units() { return g_cus; }

// A stand-in address for the scratch region (nothing is ever written there:
// launches are only recorded).
int scratch_region(void** ptr, const char**) {
    *ptr = reinterpret_cast<void*>(uintptr_t(0x5C0000000000ull));
    return 0;
}

int launch_set(const SetParams& p, void*, const char** err) {
    std::string s = p.add ? "add" : "set";
    for (int i = 0; i < p.n; ++i) s += " " + std::to_string(p.idx[i]) + "=" + std::to_string(p.val[i]);
    return record(s, err);
}

int launch_move(const MoveParams& p, void*, const char** err) {
    if (p.zero) {
        std::string s = "zero_imp";
        for (int i = 0; i < p.n; ++i)
            s += " " + std::to_string(p.sess[i]) + "@" + std::to_string(p.dst_row[i]) + "+" + std::to_string(p.rows[i]);
        return record(s, err);
    }
    std::string s = std::string(p.imp ? "move+imp" : "move");
    for (int i = 0; i < p.n; ++i)
        s += " " + std::to_string(p.sess[i]) + ":" + std::to_string(p.src_row[i]) + ">" +
             std::to_string(p.dst_row[i]) + "x" + std::to_string(p.rows[i]);
    return record(s, err);
}

int launch_append(const AppendParams& p, void*, const char** err) {
    std::string s = "append b0=" + std::to_string(p.b0) + " T=" + std::to_string(p.T) + " n=";
    for (int i = 0; i < p.nsess; ++i) s += (i ? "," : "") + std::to_string(p.n_new[i]);
    return record(s, err);
}

int launch_decode(const DecodeParams& p, void*, void* const ev[3], const char** err) {
    std::string s = std::string(ev[0] || ev[1] || ev[2] ? "traced " : "") + "decode T=" + std::to_string(p.T) + " chunk=" + std::to_string(p.chunk) +
                    " splits=" + std::to_string(p.splits) + " ml_to_o=" +
                    std::to_string((const char*)p.part_o - (const char*)p.part_ml) +
                    " kernel=" + std::to_string(p.kernel) + " gh=" + std::to_string(p.gh) +
                    " rs=" + std::to_string(p.rs) + " rg=" + std::to_string(p.rg) + " ds=" + std::to_string(p.ds) +
                    " lds=" + std::to_string(p.lds) + " units=" + std::to_string(p.units) +
                    " Tg=" + std::to_string(p.Tg) + " groups=" + std::to_string((p.T + p.Tg - 1) / p.Tg);
    return record(s, err);
}

int launch_importance(const ImportanceParams& p, void*, const char** err) {
    return record("importance T=" + std::to_string(p.T) + " tiles=" + std::to_string(p.tiles) +
                      " group_rows=" + std::to_string(p.group_rows) + " rp=" + std::to_string(p.rp),
                  err);
}

}  // namespace kvq

extern "C" {
const char* kvq_nodev_log(void) { return g_log.c_str(); }
void kvq_nodev_clear(void) { g_log.clear(); }
void kvq_nodev_fail_next(void) { g_fail_next = 1; }
void kvq_nodev_set_cus(int n) { g_cus = n; }
}
