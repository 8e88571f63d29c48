// geometry.cpp - launch geometry of the row movers and gathers.
//
// The defaults are the shapes measured fastest on MI355X (the reasons sit next
// to the launches in scatter.hip and combine.hip).  MOE_GEOM, read once when a
// launch first asks for the geometry, overrides them for tuning runs: a list of
// key=value pairs separated by commas, e.g.
//   MOE_GEOM=combine_chunk_units=224,combine_wgs_per_cu=4
// Keys and ranges are those of kFields; an unknown key, a malformed pair or a
// value outside its range is ignored and listed after "ignored:" in the text
// moe_geometry() returns.  Every value, default or override, passes this one
// range check (the launch-shape overrides of "feat(EPv2): [preview] internode
// dispatch/combine over CCO/GDA", ROCm/mori pull 625, commit log, once skipped
// a clamp and hung every rank).  The geometry decides only how work is split
// over workgroups and how many share a CU, never what is computed: results are
// the same bits under every accepted geometry.
#include <cstdlib>
#include <mutex>
#include <string>

#include "internal.hpp"

namespace moe {

namespace {

struct Field {
    const char* key;
    int Geometry::*member;
    int lo, hi;      // accepted range; a cap also accepts 0 (none)
    bool cap;
};

// combine_chunk_units: lane-units per combine workgroup (one unit per lane, at
// most 256 threads); *_wgs_per_cu: residency cap through an LDS reservation of
// 160 KB / n per workgroup, n from 3 (53 KB, within one workgroup's LDS limit)
// to 16, or 0 for none; *_chunks: workgroups per row.
constexpr Field kFields[] = {
    {"combine_chunk_units", &Geometry::combine_chunk_units, 64, 256, false},
    {"combine_wgs_per_cu", &Geometry::combine_wgs_per_cu, 3, 16, true},
    {"fp8_chunks", &Geometry::fp8_chunks, 1, 8, false},
    {"fp8_wgs_per_cu", &Geometry::fp8_wgs_per_cu, 3, 16, true},
    {"copy_chunks", &Geometry::copy_chunks, 1, 8, false},
    {"copy_wgs_per_cu", &Geometry::copy_wgs_per_cu, 3, 16, true},
    {"recv_chunks", &Geometry::recv_chunks, 1, 8, false},
    {"recv_wgs_per_cu", &Geometry::recv_wgs_per_cu, 3, 16, true},
    {"expand_chunks", &Geometry::expand_chunks, 1, 8, false},
    {"expand_wgs_per_cu", &Geometry::expand_wgs_per_cu, 3, 16, true},
};

Geometry g_geom{
    /*combine_chunk_units=*/256, /*combine_wgs_per_cu=*/5,
    /*fp8_chunks=*/2, /*fp8_wgs_per_cu=*/8,
    /*copy_chunks=*/1, /*copy_wgs_per_cu=*/0,
    /*recv_chunks=*/2, /*recv_wgs_per_cu=*/0,
    /*expand_chunks=*/1, /*expand_wgs_per_cu=*/4,
};
std::string g_text;
std::once_flag g_once;

bool parse_int(const std::string& s, int& out) {
    if (s.empty() || s.size() > 9) return false;
    int v = 0;
    for (char ch : s) {
        if (ch < '0' || ch > '9') return false;
        v = v * 10 + (ch - '0');
    }
    out = v;
    return true;
}

void init() {
    std::string ignored;
    if (const char* env = std::getenv("MOE_GEOM")) {
        const std::string spec(env);
        size_t pos = 0;
        while (pos <= spec.size()) {
            size_t end = spec.find(',', pos);
            if (end == std::string::npos) end = spec.size();
            const std::string item = spec.substr(pos, end - pos);
            pos = end + 1;
            if (item.empty()) continue;
            const size_t eq = item.find('=');
            bool ok = false;
            if (eq != std::string::npos) {
                const std::string key = item.substr(0, eq);
                int v = 0;
                if (parse_int(item.substr(eq + 1), v)) {
                    for (const Field& f : kFields) {
                        if (key == f.key && ((v >= f.lo && v <= f.hi) || (f.cap && v == 0))) {
                            g_geom.*(f.member) = v;
                            ok = true;
                        }
                    }
                }
            }
            if (!ok) ignored += (ignored.empty() ? "" : ",") + item;
        }
    }
    for (const Field& f : kFields) {
        if (!g_text.empty()) g_text += ",";
        g_text += std::string(f.key) + "=" + std::to_string(g_geom.*(f.member));
    }
    if (!ignored.empty()) g_text += "; ignored: " + ignored;
}

}  // namespace

const Geometry& geometry() {
    std::call_once(g_once, init);
    return g_geom;
}

const char* geometry_text() {
    std::call_once(g_once, init);
    return g_text.c_str();
}

}  // namespace moe
