// Launchers for the host-only build of libbkv (argument checks, workspace sizing and the
// overlap sweep of bkv_api.hip, built with host sanitizers for CPU tests).  That build
// holds no kernels: every launcher refuses, so a call that passes validation returns
// BKV_EHIP instead of enqueuing anything.
#include "bkv_internal.h"

namespace bkv {

static hipError_t refuse(const char* what) { return note_hip_error(hipErrorNotSupported, what); }

hipError_t launch_score(const ScoreArgs&, int, int, hipStream_t) { return refuse("host-only build: score"); }
bool qs_stats_covers(int, int) { return false; }
hipError_t qs_stats_occupancy(int, int, int*) { return refuse("host-only build: score occupancy"); }
hipError_t launch_qs_stats(const ScoreArgs&, int, int, hipStream_t) { return refuse("host-only build: score"); }
hipError_t launch_select(const SelectArgs&, int, hipStream_t) { return refuse("host-only build: select"); }
hipError_t launch_compact(const CompactArgs&, int, int, hipStream_t) { return refuse("host-only build: compact"); }
hipError_t launch_decode(const DecodeArgs&, int, int, hipStream_t) { return refuse("host-only build: decode"); }
hipError_t launch_fps(const FpsArgs&, int, int, int, hipStream_t) { return refuse("host-only build: fps"); }
hipError_t launch_initial(const FpsArgs&, int, int, hipStream_t) { return refuse("host-only build: fps"); }

}  // namespace bkv
