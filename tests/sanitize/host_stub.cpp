// Host-only stand-in for the one device query the planners make, so that the validation
// and planning code (wq_validate.cpp, wq_plan.cpp) links into a library without the HIP
// runtime: a sanitizer build of exactly that code, driven by the validation tests.
namespace wq {
int device_cu_count() { return 256; }
}  // namespace wq
