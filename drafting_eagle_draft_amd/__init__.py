"""MI355X-native (gfx950) P-EAGLE parallel-drafter hot path.

libpeagle.so (built from csrc/ by ``python -m drafting_eagle_draft_amd.build``)
holds every kernel; ``binding`` is its ctypes binding, ``runner`` the device
buffer helpers, ``synth`` the seeded synthetic inputs.  Importing the package
loads nothing; the binding loads the library on first use and raises if it
is missing.
"""
__all__ = ["binding", "runner", "synth", "build"]
