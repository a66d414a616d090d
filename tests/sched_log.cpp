// Host-only driver of the DBO schedule (dbo_schedule.h) on a recording
// backend: prints every operation the schedule issues so the Python test can
// rebuild the happens-before graph.  Usage: sched_log <schedule> <fail_at|-1>
#include <cstdio>
#include <cstdlib>

#include "dbo_schedule.h"

using namespace dbomoe::sched;

struct Recorder {
  int n = 0;
  int fail_at = -1;
  int step() { return n++ == fail_at ? -5 : 0; }
  int launch(int s, int mb, int st) {
    const int r = step();
    if (r == 0) std::printf("LAUNCH %d %d %d\n", s, mb, st);
    return r;
  }
  int record(int s, int ev) {
    const int r = step();
    if (r == 0) std::printf("RECORD %d %d\n", s, ev);
    return r;
  }
  int wait(int s, int ev) {
    const int r = step();
    if (r == 0) std::printf("WAIT %d %d\n", s, ev);
    return r;
  }
  int join() {
    std::printf("JOIN\n");
    return 0;
  }
};

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  const int schedule = std::atoi(argv[1]);
  Recorder rec;
  rec.fail_at = std::atoi(argv[2]);
  const Plan plan = build_plan(schedule);
  RunStats st;
  const int status = run_plan(plan, rec, &st);
  std::printf("YIELDS %d %d\n", st.yields[0], st.yields[1]);
  std::printf("STATUS %d\n", status);
  return 0;
}
